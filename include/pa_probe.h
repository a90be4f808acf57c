/*
 * pa_probe.h - read-bandwidth probes for libpa.so (AMD Instinct MI355X,
 * gfx950).  C ABI; include pa.h first.
 *
 * They measure the practical ceilings a paged decode is held against: the
 * rate of a plain streaming read, and the rate of the decode's own loads
 * with no arithmetic (the cache is a pool of blocks reached through each
 * sequence's block table: "Taming the token torrent", "The Block Table
 * Logic").  They are measurement tools, not steps of the decode.
 *
 * Both fold every 32-bit word they read into *sink with XOR (one device
 * uint32 the caller zeroes beforehand; calls accumulate), so their loads
 * cannot be optimised away and the bytes read can be checked.
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16, 16-byte aligned) of DEVICE memory at buf
 * once, front to back in grid-strided 16-byte loads.  *sink ^= XOR of all
 * its 32-bit words.  PA_ERR_NULL, PA_ERR_SHAPE for a size or alignment that
 * is not a multiple of 16, PA_ERR_DEVICE without a gfx950.                  */
pa_status pa_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Reads what pa_decode_window (bf16 cache, elem_bytes 2) or
 * pa_decode_window_fp8 (elem_bytes 1) reads of the caches for the same
 * arguments (window 0: what pa_decode / pa_decode_fp8 read): for every
 * sequence s with 1 <= L = seq_lens[s] <= max_blocks_per_seq * block_size
 * and KV head h, the K and V tiles of 16 tokens covering tokens
 * [max(0, L - window), L) (window > 0) or [0, L) (window 0) through
 * block_tables (block ids outside the pool are skipped; table entries of
 * tiles before the window are not read).  *sink ^= XOR of all 32-bit words
 * of those tiles, each tile counted once per (sequence, head) that reads it.
 * Validation as pa_decode's (PA_ERR_UNSUPPORTED for elem_bytes other than 1
 * and 2; PA_ERR_SHAPE for window < 0).                                     */
pa_status pa_probe_tile_read(const pa_cache_desc* cache, int32_t elem_bytes, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables, int32_t num_seqs,
                             int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t window,
                             uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
