// Internal declarations shared by the HIP translation units of libpa.so.
// Nothing here is part of the C ABI (see include/pa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Tokens per cache sub-block: the unit one wavefront's MFMA tile covers.
constexpr int kSub = 16;
// Wavefronts per workgroup of the decode kernel (independent of each other).
#ifndef PA_DECODE_WAVES_PER_GROUP
#define PA_DECODE_WAVES_PER_GROUP 4
#endif
constexpr int kWavesPerGroup = PA_DECODE_WAVES_PER_GROUP;
constexpr int kDecodeThreads = 64 * kWavesPerGroup;

// e4m3fn code of float32(x * inv): round to nearest even, saturate to
// +-448, NaN -> 0x7F with x's sign ("KV Cache Engineering for LLM Serving",
// section 8, Quantization: divide by the scale, round, clip).  Clamping
// first keeps the hardware conversion inside the finite range, where it
// rounds to nearest even (a NaN clamps to -448 and its code is replaced).
// Branch-free, so loops over it unroll into straight-line code.
__device__ __forceinline__ uint32_t e4m3_code(float x, float inv) {
  float y = x * inv;
  y = __builtin_fminf(__builtin_fmaxf(y, -448.0f), 448.0f);
  const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFFu;
  const uint32_t nan_code = (__float_as_uint(x) >> 24 & 0x80u) | 0x7Fu;
  return __builtin_isnan(x) ? nan_code : code;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Element index of V (token r of a 16-token tile, dim d) inside its tile:
// [d / 16R][d % 16][r / 4][(d / 16) % R][r % 4].
template <int R>
__device__ __forceinline__ int v_elem(int d, int r) {
  return ((((d / (16 * R)) * 16 + d % 16) * 4 + r / 4) * R + (d / 16) % R) * 4 + r % 4;
}

// Query-aware page summaries: one uint32 word per (block, KV head, key
// dimension), (max bf16 << 16) | min bf16, laid out [block][d / 4][head][4]
// so that the 16-byte quads of all heads for 4 dimensions of a block are
// contiguous (the score kernel reads one such run per page and step).
__host__ __device__ __forceinline__ int64_t summary_word(int64_t blk, int h, int d, int num_kv_heads, int head_dim) {
  return ((blk * (head_dim / 4) + d / 4) * num_kv_heads + h) * 4 + d % 4;
}
constexpr uint32_t kEmptySummaryWord = 0xFF807F80u;  // max = -inf (bf16 0xFF80), min = +inf (0x7F80)

struct CacheWriteParams {
  const uint16_t* k;          // [T][Hkv][D] bf16 bits
  const uint16_t* v;
  const int64_t* slots;       // [T]
  uint8_t* k_cache;
  uint8_t* v_cache;
  uint32_t* summaries;        // null, or the pool's page summaries, kept current by the write
  int32_t num_tokens, num_kv_heads, head_dim, block_size;
  int64_t num_slots;          // num_blocks * block_size
  float k_inv, v_inv;         // 1 / scale (fp8 only)
};

struct DecodeParams {
  const uint16_t* q;          // [S][Hq][D] bf16 bits
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;  // [S][max_blocks]
  const int32_t* seq_lens;      // [S]
  float* out;                   // [S][Hq][D]
  float* lse;                   // null, or [S][Hq]: log2 of each row's softmax sum in logit
                                // units of qk_scale (m + log2 l); -inf for empty rows
  float* partials;              // [2 * num_waves][G * (D + 4)]
  int32_t* counters;            // [S * Hkv] pieces (or groups) counted in per unit; zero between calls
  int32_t* group_counters;      // null, or [kGroupCounters] pieces counted in per merge-tree group,
                                // indexed by the record slot of the group's first piece; zero
                                // between calls
  int32_t num_seqs, num_q_heads, num_kv_heads, group, head_dim, block_size, num_blocks, max_blocks;
  int32_t num_waves;            // wavefronts launched
  int32_t chunk_min;            // auto split: fewest chunks a wavefront takes
  int32_t chunk_fixed;          // > 0: every wavefront takes this many chunks
  int32_t unit_charge;          // auto split: chunks each unit counts for beyond its own (0 with
                                // fixed partitions)
  int32_t window;               // > 0: attend to the last `window` tokens only
  int32_t ring;                 // != 0: each table row is a ring of max_blocks entries, logical
                                // block b at entry b % max_blocks (local layers, window > 0)
  int32_t subs;                 // 16-token sub-blocks per block (block_size / 16)
  uint32_t subs_magic;          // ceil(2^32 / subs) for subs > 1: j / subs = umulhi(j, magic)
  int64_t blk_stride;           // bytes from one block's tiles to the next: Hkv * subs * tile
  int32_t seq_heads;            // > 1: sequence s reads KV head s % seq_heads (one KV head per
                                // sequence; its tables are per (sequence, head))
  uint32_t seq_heads_magic;     // ceil(2^32 / seq_heads): s / seq_heads = umulhi(s, magic)
  float qk_scale;               // scale * log2(e) (* k_scale for fp8)
  float out_scale;              // 1 (bf16) or v_scale (fp8)
  // Fused append (all null otherwise): sequence s's new token, rows
  // [s][h][:] of k_new / v_new ([S][Hkv][D] bf16), is position L - 1; it is
  // stored into the caches (k_store / v_store, the same memory as k_cache /
  // v_cache) and attended to from registers.
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint8_t* k_store;
  uint8_t* v_store;
  float k_inv, v_inv;           // fp8 append: 1 / k_scale, 1 / v_scale
};

struct BlockMoveParams {
  const uint8_t* src_k;         // source buffers (caches, or pinned host memory)
  const uint8_t* src_v;
  uint8_t* dst_k;               // destination buffers
  uint8_t* dst_v;
  const int32_t* src_ids;       // item i reads block src_ids[i * id_stride] (null: block i)
  const int32_t* dst_ids;       // item i writes block dst_ids[i * id_stride] (null: block i)
  int64_t block_bytes;          // Hkv * block_size * head_dim * element bytes
  int32_t id_stride;
  int32_t segs;                 // 16 KiB segments per block (the last may be shorter)
  int32_t last_words;           // 16-byte words in a block's last segment
  int32_t num_items, src_blocks, dst_blocks;
};

// Query-aware page selection: largest query group the score kernel takes.
constexpr int kMaxGroupQuest = 16;

struct SummaryParams {
  const uint8_t* k_cache;
  const int64_t* slots;         // update: [num_tokens] slots just written
  const int32_t* blocks;        // build: [num_tokens] blocks to recompute ...
  const int32_t* counts;        // ... from their first counts[i] tokens
  uint32_t* words;              // summaries, laid out as summary_word() says
  int32_t num_tokens;           // tokens (update) or listed blocks (build)
  int32_t num_kv_heads, head_dim, block_size, num_blocks;
};

struct SelectParams {
  const uint16_t* q;            // [S][Hq][D] bf16 bits
  const uint32_t* words;        // summaries
  const int32_t* block_tables;  // [S][max_blocks]
  const int32_t* seq_lens;      // [S]
  uint32_t* keys;               // workspace [S * Hkv][max_blocks] page score keys
  int32_t* sel_tables;          // [S * Hkv][budget]
  int32_t* sel_lens;            // [S * Hkv]
  int32_t num_seqs, num_q_heads, num_kv_heads, group, head_dim, block_size, num_blocks, max_blocks;
  int32_t budget;               // pages to keep per (sequence, KV head)
  int32_t slice_heads;          // KV heads whose queries a score workgroup holds at once
  int32_t item_pages;           // pages a score workgroup takes per item
};

// Shared-prefix decode: attention over shared segments for all their members.
struct SegmentParams {
  const uint16_t* q;            // [S][Hq][D] bf16 bits
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* items;         // [num_items][8]: blocks offset, blocks, members offset, members,
                                //                 KV head, first partial slot, 0, 0
  const int32_t* seg_blocks;    // block ids of every segment chunk
  const int32_t* members;       // member sequence ids
  float* partials;              // [slots][Hq][D + 4]: acc[D], m, l, 0, 0 (base-2 logits)
  int32_t num_items, num_q_heads, group, mpw, head_dim, block_size, num_blocks;
  int32_t num_seqs, num_slots;  // members and slots outside these are skipped
  int64_t blk_stride;           // bytes from one block's tiles to the next
  float qk_scale;               // |scale| * log2(e) (* k_scale for fp8), never negative
  uint32_t q_sign;              // 0x80008000 when scale < 0: q is negated as it is loaded
};

struct TileProbeParams {
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;  // [num_seqs][max_blocks]
  const int32_t* seq_lens;
  uint32_t* sink;               // XOR of every word read is folded in
  int32_t num_seqs, num_kv_heads, max_blocks, block_size, num_blocks, head_dim, elem_bytes;
  int32_t window;               // > 0: only the tiles of the last `window` tokens
  int64_t blk_stride;           // bytes per block of one cache
};

struct CombineParams {
  const float* part_out;        // [S][Hq][D] private part, normalized and scaled
  const float* part_lse;        // [S][Hq] its log2-sum-exp (-inf when empty)
  const float* partials;        // shared parts
  const int32_t* parts_off;     // [S + 1] into parts
  const int32_t* parts;         // partial slots of each sequence
  float* out;
  int32_t num_seqs, num_q_heads, head_dim, num_slots;   // a slot outside num_slots makes the row NaN
  float out_scale;              // 1 (bf16) or v_scale (fp8), applied to the shared parts
};

// Host-side launchers (defined next to their kernels).
hipError_t launch_cache_write(const CacheWriteParams& p, bool fp8, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, bool fp8, hipStream_t stream);
hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t stream);
// max_groups > 0 caps the grid (the workgroups then stride over the
// segments); 0 launches one workgroup per segment.
hipError_t launch_move_blocks(const BlockMoveParams& p, int max_groups, hipStream_t stream);
hipError_t launch_summary_fill(uint32_t* words, int64_t n_words, hipStream_t stream);
hipError_t launch_summary_update(const SummaryParams& p, bool fp8, hipStream_t stream);
hipError_t launch_summary_build(const SummaryParams& p, bool fp8, hipStream_t stream);
hipError_t launch_page_select(const SelectParams& p, hipStream_t stream);
hipError_t launch_segments(const SegmentParams& p, bool fp8, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int grid, hipStream_t stream);
hipError_t launch_tile_read(const TileProbeParams& p, int grid, hipStream_t stream);
// Resident wavefronts of the decode kernel on the current device (0 on error).
int decode_resident_waves(int head_dim, bool fp8);

// Workspace carve-up shared by the size query and the launchers.  The
// per-unit counters come first, in a region of at least kMinCounterUnits
// entries, then kGroupCounters counters of the merge tree's groups (indexed
// by record slot): for every call with num_seqs * num_kv_heads <=
// kMinCounterUnits the counters then occupy the same first 128 KiB, which
// nothing else in the workspace is ever used for, whatever the other sizes
// (wave count, group, head_dim, partition) of the calls sharing it.  Each
// call leaves its counters at zero, so such calls can share one workspace
// that was zero-filled once.  The partial records follow; they are always
// written before they are read, so their contents between calls do not
// matter.
constexpr int64_t kMinCounterUnits = 16384;
constexpr int64_t kGroupCounters = 16384;   // record slots (2 per wavefront) the tree can count
struct WorkspaceLayout {
  size_t counters_off, group_counters_off, partials_off, total;
};
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline size_t counter_region_bytes(int64_t units) {
  return align_up((size_t)(units > kMinCounterUnits ? units : kMinCounterUnits) * sizeof(int32_t), 256);
}
inline WorkspaceLayout workspace_layout(int64_t num_waves, int group, int head_dim,
                                        int num_seqs, int num_kv_heads) {
  WorkspaceLayout w;
  w.counters_off = 0;
  w.group_counters_off = counter_region_bytes((int64_t)num_seqs * num_kv_heads);
  w.partials_off = w.group_counters_off + (size_t)kGroupCounters * sizeof(int32_t);
  const size_t part = (size_t)(2 * num_waves) * (size_t)group * (size_t)(head_dim + 4) * sizeof(float);
  w.total = align_up(w.partials_off + part, 256);
  return w;
}

}  // namespace pa
