/*
 * pa_blocks.h - block manager and block copies for the paged KV cache of
 * libpa.so (AMD Instinct MI355X, gfx950).  C ABI; include pa.h first.
 *
 * The block manager is the host-side step just before the decode path: it
 * hands out physical blocks, builds each sequence's block table, produces the
 * slot of every new token for pa_cache_write, and shares blocks between
 * sequences with identical prefixes.  Its rules, from the pages:
 *   - The pool is a list of free block ids.  A request takes blocks from the
 *     front; a finished request returns its blocks to the back in the order of
 *     its block table, ready for the next request ("KV Cache Engineering for
 *     LLM Serving", section 10, Paging).
 *   - A completed block is kept under a key made of the whole token prefix up
 *     to its end, so it is reused only when all preceding context is
 *     identical; the key also holds a model / adapter identity (same page,
 *     section 11, Prefix reuse; rajatmohan.com serving design, "Prefix sharing
 *     is where the real win lives").  Keys are compared exactly (the prefix
 *     is interned), so there are no hash collisions.
 *   - A reused block's reference count is incremented; a sequence that writes
 *     into a block someone else still holds first gets a private copy
 *     (copy-on-write; "Taming the token torrent", "Implementing Radix Tree
 *     Prefix Caching").
 * Only full blocks are ever shared by key; a partly filled last block is
 * private, unless the sequence was forked (parallel sampling, beam search),
 * in which case the first append to it copies it.
 *
 * The manager is host memory only, not thread-safe (one caller at a time per
 * manager), and never touches the GPU: block copies it asks for are done with
 * pa_copy_blocks on the caller's stream before the step's pa_cache_write.
 */
#ifndef PA_BLOCKS_H_
#define PA_BLOCKS_H_

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A manager of num_blocks blocks of block_size tokens (both >= 1), all free,
 * ids 0..num_blocks-1 in the free list in that order.  *out receives the
 * handle (NULL on error).                                                    */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager** out);

/* Frees the manager; NULL is a no-op.                                        */
void pa_bm_destroy(pa_block_manager* bm);

/* A new sequence `seq` with prompt tokens[0..n) (n >= 0) under model key
 * `model_key`.  Every full block whose prefix key is stored is reused
 * (reference count + 1); the other full blocks and a partial last block are
 * taken from the free list, and the new full blocks are stored under their
 * keys.  *reused (may be NULL) receives the number of reused blocks.
 * PA_ERR_NOT_FOUND if seq already exists; PA_ERR_NO_BLOCKS, with nothing
 * changed, if the free list is too short.                                    */
pa_status pa_bm_add_sequence(pa_block_manager* bm, int64_t seq, const int32_t* tokens,
                             int32_t n, uint64_t model_key, int32_t* reused);

/* A local layer's sequence with a ring table ("KV Cache Engineering for LLM
 * Serving", section 3, sliding windows: a local layer keeps its most recent
 * `window` positions only, each new one displacing the oldest).  The table
 * has *ring_entries = ceil(window / block_size) + 1 entries, and logical
 * block b (positions b * block_size ..) is entry b % ring_entries, so a
 * window's blocks never share an entry.  The sequence starts with n tokens
 * (n >= 0, a prompt whose K/V the caller writes to the slots pa_bm_slots
 * gives): blocks are taken for its last min(ceil(n / block_size),
 * ring_entries) logical blocks, the other entries are -1.  Afterwards
 * pa_bm_append_token (its `token` argument is not kept) fills the ring:
 * where a new block starts, the entry's old block, which has left the
 * window, is written over in place when no other sequence holds it, so a
 * full ring takes no more blocks from the pool; a block a fork still shares
 * is let go and a fresh one taken, and a shared partial block is copied
 * first as for plain tables.  Ring sequences keep no token ids and share no
 * prefix blocks.  Use pa_decode_ring on their tables; pa_bm_batch needs
 * max_blocks == ring_entries for them.  window >= 1, else PA_ERR_SHAPE;
 * PA_ERR_NOT_FOUND if seq exists; PA_ERR_NO_BLOCKS, with nothing changed,
 * if the free list is too short.                                            */
pa_status pa_bm_add_ring_sequence(pa_block_manager* bm, int64_t seq, int32_t n, int32_t window,
                                  int32_t* ring_entries);

/* Slots of positions first .. first + count - 1 of `seq` (plain or ring):
 * slots[i] = block * block_size + offset of position first + i, or -1 when
 * the sequence holds no block for it any more (a trimmed entry, or a ring
 * entry that has moved on).  PA_ERR_SHAPE unless 0 <= first, 0 <= count and
 * first + count <= the sequence's token count; PA_ERR_SWAPPED while the
 * sequence is swapped out.                                                  */
pa_status pa_bm_slots(const pa_block_manager* bm, int64_t seq, int32_t first, int32_t count,
                      int64_t* slots);

/* Sequence `child` shares every block of `parent` (reference counts + 1),
 * with the same tokens and model key.  PA_ERR_NOT_FOUND if parent is unknown
 * or child exists.                                                           */
pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);

/* Appends one token to `seq`.  *slot receives the physical slot (block *
 * block_size + offset) its K/V go to.  When the token starts a new block a
 * block is taken from the free list; when it lands in a partial block that
 * other sequences still hold, a fresh block replaces it in this sequence's
 * table and (*copy_src, *copy_dst) name the copy to make before the write;
 * otherwise both are -1.  A block completed by the token is stored under its
 * prefix key unless an equal block is already stored.  PA_ERR_NO_BLOCKS,
 * with nothing changed, if a block is needed and none is free.               */
pa_status pa_bm_append_token(pa_block_manager* bm, int64_t seq, int32_t token, int64_t* slot,
                             int32_t* copy_src, int32_t* copy_dst);

/* Ends `seq`: each block of its table, in order, loses one reference; a
 * block left with none drops its key and goes to the back of the free list. */
pa_status pa_bm_free_sequence(pa_block_manager* bm, int64_t seq);

/* Sliding window ("KV Cache Engineering for LLM Serving", section 3): the
 * blocks of `seq` that hold only positions before its last keep_tokens
 * tokens (keep_tokens >= 1) each lose one reference, and their table entries
 * become -1; the table keeps its length, so later positions keep their
 * logical blocks.  pa_decode_window with window <= keep_tokens never reads
 * the released entries.  *released (may be NULL) receives the count.  On a
 * ring sequence the same holds for the blocks its ring still lists.        */
pa_status pa_bm_trim(pa_block_manager* bm, int64_t seq, int32_t keep_tokens, int32_t* released);

/* Swap-out bookkeeping: the blocks of `seq` that no other sequence holds
 * (reference count 1) are listed, in table order, in blocks[0..*n) and
 * released to the free list (their keys dropped); their table entries become
 * -2 (swapped).  Shared blocks stay with the sequence, since a prefix other
 * sequences use is the last thing to move out ("Taming the token torrent",
 * "The Swapping Mechanism").  The caller copies the listed blocks out with
 * pa_swap_out on its stream before anything it enqueues later can write
 * them.  A swapped sequence cannot be appended to, forked, trimmed or
 * batched until pa_bm_swap_in (PA_ERR_SWAPPED).  PA_ERR_SHAPE, with nothing
 * changed, if more than `capacity` blocks would be listed.                   */
pa_status pa_bm_swap_out(pa_block_manager* bm, int64_t seq, int32_t* blocks, int32_t capacity,
                         int32_t* n);

/* Swap-in bookkeeping: each swapped entry of `seq`, in table order, gets a
 * block from the free list, listed in blocks[0..*n) in the same order as
 * pa_bm_swap_out listed the blocks it replaced, so the host copy's i-th
 * block goes to blocks[i] (pa_swap_in).  A full block is stored under its
 * prefix key again unless an equal block is stored.  PA_ERR_NO_BLOCKS or
 * PA_ERR_SHAPE (capacity), with nothing changed; PA_ERR_SWAPPED if `seq` is
 * not swapped out.                                                          */
pa_status pa_bm_swap_in(pa_block_manager* bm, int64_t seq, int32_t* blocks, int32_t capacity,
                        int32_t* n);

/* Free blocks (or -1 for a NULL manager).                                    */
int32_t pa_bm_num_free(const pa_block_manager* bm);

/* Token count and block count (table length, released entries included) of
 * `seq`.                                                                     */
pa_status pa_bm_sequence_info(const pa_block_manager* bm, int64_t seq, int32_t* num_tokens,
                              int32_t* num_blocks);

/* Copies the block table of `seq` into out[0..capacity); PA_ERR_SHAPE if it
 * has more than `capacity` blocks.                                           */
pa_status pa_bm_block_table(const pa_block_manager* bm, int64_t seq, int32_t* out,
                            int32_t capacity);

/* Reference count of `block` (0 when free).                                  */
pa_status pa_bm_refcount(const pa_block_manager* bm, int32_t block, int32_t* ref);

/* Reused and newly taken full-or-partial blocks over all add_sequence calls. */
pa_status pa_bm_stats(const pa_block_manager* bm, int64_t* hits, int64_t* misses);

/* Host arrays for one decode batch of the sequences seqs[0..n):
 * block_tables[n][max_blocks] (entries past a sequence's blocks set to -1)
 * and seq_lens[n] (token counts).  PA_ERR_SHAPE if a sequence has more than
 * max_blocks blocks, or is a ring sequence with ring_entries != max_blocks
 * (its row must be the ring itself).                                        */
pa_status pa_bm_batch(const pa_block_manager* bm, const int64_t* seqs, int32_t n,
                      int32_t max_blocks, int32_t* block_tables, int32_t* seq_lens);

/* Copies whole blocks of both caches on the GPU: for each i < num_pairs,
 * block pairs[2i+1] of k_cache and v_cache becomes a bit copy of block
 * pairs[2i] (every KV head, every token slot).  In the cache layout of pa.h a
 * block is one contiguous run of num_kv_heads * block_size * head_dim
 * elements of elem_bytes bytes (2 for bf16, 1 for fp8).
 *   pairs      DEVICE array [num_pairs][2] int32 {src, dst}
 * Pairs must be independent (no block is the destination of two pairs or
 * both a source and a destination); pairs with an id outside
 * [0, num_blocks) are skipped.  num_pairs == 0 is a no-op.  The copy-on-write
 * pairs of pa_bm_append_token always satisfy this.                          */
pa_status pa_copy_blocks(const pa_cache_desc* cache, int32_t elem_bytes, void* k_cache,
                         void* v_cache, const int32_t* pairs, int32_t num_pairs, void* stream);

/* Swap blocks out to host memory: blocks[i] of k_cache and v_cache (for
 * i < num_blocks; DEVICE int32 array) are copied into `host`, which holds the
 * K blocks in list order, then the V blocks: 2 * num_blocks * block_bytes
 * bytes, block_bytes = num_kv_heads * block_size * head_dim * elem_bytes.
 * `host` must be pinned memory from hipHostMalloc (any offset into such an
 * allocation), else PA_ERR_HOST_MEMORY: a kernel on `stream` writes it
 * directly through its device mapping, so there is no staging buffer and no
 * separate DMA step.  The call returns without waiting; the host copy is
 * complete when the stream's work is.  Ids outside [0, num_blocks of the
 * cache) are skipped (their slots of `host` are left as they were).  The
 * kernel occupies a small fixed grid, so it can run on a second stream
 * beside decode work on another ("Taming the token torrent", "The Swapping
 * Mechanism": the copy back is hidden under the first layers' work).        */
pa_status pa_swap_out(const pa_cache_desc* cache, int32_t elem_bytes, const void* k_cache,
                      const void* v_cache, const int32_t* blocks, int32_t num_blocks, void* host,
                      void* stream);

/* Swap blocks back in: the reverse of pa_swap_out.  The i-th K and V blocks
 * of `host` (pinned, laid out as pa_swap_out writes it) become blocks[i] of
 * k_cache and v_cache; ids outside [0, num_blocks of the cache) are skipped.
 * The host buffer must not change until the stream's work is complete.     */
pa_status pa_swap_in(const pa_cache_desc* cache, int32_t elem_bytes, void* k_cache, void* v_cache,
                     const int32_t* blocks, int32_t num_blocks, const void* host, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H_ */
