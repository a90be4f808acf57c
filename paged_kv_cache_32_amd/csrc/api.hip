// extern "C" entry points of libpa.so: host-side validation, workspace
// sizing and kernel launches.  See include/pa.h for the contract.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/pa.h"
#include "../../include/pa_blocks.h"
#include "../../include/pa_quest.h"
#include "../../include/pa_cascade.h"
#include "../../include/pa_probe.h"
#include "pa_internal.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxGroup = 16;
constexpr int kMaxBlockSize = 256;
// Chunks each unit counts for beyond its own in the automatic split (its
// fixed costs: the sequence's length and table entries, the query, a
// partial record).  They pay on the fp8 cache, where a chunk is half the
// bytes; on bf16 the split by chunks alone measured best.
#ifndef PA_DECODE_UNIT_CHARGE
#define PA_DECODE_UNIT_CHARGE 0
#endif
#ifndef PA_DECODE_UNIT_CHARGE_FP8
#define PA_DECODE_UNIT_CHARGE_FP8 4
#endif
// The shared-prefix decode's private parts on a bf16 cache: thousands of
// short units (each sequence's blocks after its shared prefix, for every KV
// head), where the per-unit charge pays (measured 600 against 618-625 us
// per call on the 256-sequence prefix-shared batch, on two machines).
#ifndef PA_CASCADE_UNIT_CHARGE
#define PA_CASCADE_UNIT_CHARGE 2
#endif
// Fewest chunks a wavefront takes in the automatic split.  It only binds on
// short reads (fewer chunks than 8 per resident wavefront); there more,
// shorter pieces win now that a long unit's pieces merge as a tree.
#ifndef PA_DECODE_CHUNK_MIN
#define PA_DECODE_CHUNK_MIN 8
#endif
constexpr int kChunkMinAuto = PA_DECODE_CHUNK_MIN;  // fewest chunks per wavefront when splitting automatically
// Wavefronts launched per resident slot in the automatic split: ranges left
// over are picked up by whichever slots free up first.
#ifndef PA_DECODE_OVERSUB
#define PA_DECODE_OVERSUB 1
#endif
// Workgroups of a swap to or from host memory.  Each keeps 16 KiB of
// requests in flight; 8 of them (128 KiB) keep the host link at 51-57 GB/s
// on MI355X.  More add no throughput: the extra requests only queue in the
// memory system, where they hold up the HBM reads of a decode running beside
// the swap (measured: a 64 MiB swap-out next to the 70B-layer decode slows
// it 1.6x at 8 workgroups, 5x at 16 or more).
#ifndef PA_SWAP_GROUPS
#define PA_SWAP_GROUPS 8
#endif

struct DeviceInfo {
  bool queried = false;
  bool gfx950 = false;
  int resident[2][2] = {{0, 0}, {0, 0}};  // [head_dim == 128][fp8]
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_mu;

// Is the current device a gfx950, and how many decode wavefronts fit on it?
bool device_info(int head_dim, bool fp8, int* resident) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.queried) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.queried = true;
  }
  if (!d.gfx950) return false;
  int& r = d.resident[head_dim == 128][fp8];
  if (r == 0) r = pa::decode_resident_waves(head_dim, fp8);
  *resident = r;
  return r > 0;
}

bool valid_desc(const pa_cache_desc* c) {
  return c->num_blocks >= 1 && c->num_kv_heads >= 1 && c->block_size >= pa::kSub &&
         c->block_size <= kMaxBlockSize && c->block_size % pa::kSub == 0 &&
         (c->head_dim == 64 || c->head_dim == 128);
}

pa_status desc_status(const pa_cache_desc* c) {
  if (c->num_blocks < 1 || c->num_kv_heads < 1 || c->block_size < 1 || c->head_dim < 1)
    return PA_ERR_SHAPE;
  if (!valid_desc(c)) return PA_ERR_UNSUPPORTED;
  // Element offsets must fit in 63 bits with room to spare.
  const double elems = (double)c->num_blocks * c->num_kv_heads * c->block_size * c->head_dim;
  if (elems > 4.0e18) return PA_ERR_SHAPE;
  return PA_OK;
}

bool good_scale(float s) { return isfinite(s) && s > 0.f; }

pa_status cache_write(const pa_cache_desc* cache, const void* k, const void* v,
                      const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                      void* v_cache, bool fp8, float k_scale, float v_scale, void* stream,
                      uint32_t* summaries = nullptr) {
  if (!cache) return PA_ERR_NULL;
  pa_status st = desc_status(cache);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (fp8 && (!good_scale(k_scale) || !good_scale(v_scale))) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
  int resident = 0;
  if (!device_info(cache->head_dim, fp8, &resident)) return PA_ERR_DEVICE;
  pa::CacheWriteParams p;
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.slots = slot_mapping;
  p.k_cache = static_cast<uint8_t*>(k_cache);
  p.v_cache = static_cast<uint8_t*>(v_cache);
  p.summaries = summaries;
  p.num_tokens = num_tokens;
  p.num_kv_heads = cache->num_kv_heads;
  p.head_dim = cache->head_dim;
  p.block_size = cache->block_size;
  p.num_slots = (int64_t)cache->num_blocks * cache->block_size;
  // Correctly rounded float32 reciprocals (IEEE division on the host).
  volatile float one = 1.0f;
  p.k_inv = fp8 ? one / k_scale : 1.0f;
  p.v_inv = fp8 ? one / v_scale : 1.0f;
  if (pa::launch_cache_write(p, fp8, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

// Wavefronts to launch and the fixed chunk count per wavefront (0 = auto).
// With fixed partitions the wavefront count covers an upper bound of the
// chunks: every sequence's whole table, or with a window of W tokens at most
// (W + 15) / 16 + 1 chunks per sequence.
pa_status plan(const pa_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
               int32_t max_blocks_per_seq, int32_t partition_tokens, bool fp8,
               int64_t* num_waves, int32_t* chunk_fixed, int32_t window = 0) {
  if (!c) return PA_ERR_NULL;
  pa_status st = desc_status(c);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads < 1 || max_blocks_per_seq < 0) return PA_ERR_SHAPE;
  if (num_q_heads % c->num_kv_heads != 0) return PA_ERR_SHAPE;
  if (num_q_heads / c->num_kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (partition_tokens < 0 || partition_tokens % pa::kSub != 0) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * c->block_size > INT32_MAX) return PA_ERR_SHAPE;
  // Every index of the kernel's chunk list must fit an int (with headroom).
  {
    const int64_t chunks_per_seq = ((int64_t)max_blocks_per_seq * c->block_size + pa::kSub - 1) / pa::kSub;
    if ((int64_t)num_seqs * c->num_kv_heads * chunks_per_seq >= ((int64_t)1 << 30)) return PA_ERR_SHAPE;
  }
  int resident = 0;
  if (!device_info(c->head_dim, fp8, &resident)) return PA_ERR_DEVICE;
  if (partition_tokens == 0) {
    *num_waves = (int64_t)resident * PA_DECODE_OVERSUB;
    *chunk_fixed = 0;
  } else {
    const int64_t per = partition_tokens / pa::kSub;
    int64_t chunks_per_seq = ((int64_t)max_blocks_per_seq * c->block_size + pa::kSub - 1) / pa::kSub;
    if (window > 0 && ((int64_t)window + pa::kSub - 1) / pa::kSub + 1 < chunks_per_seq)
      chunks_per_seq = ((int64_t)window + pa::kSub - 1) / pa::kSub + 1;
    const int64_t upper = (int64_t)num_seqs * c->num_kv_heads * chunks_per_seq;
    int64_t w = (upper + per - 1) / per;
    if (w < 1) w = 1;
    if (w > (int64_t)INT32_MAX - pa::kWavesPerGroup) return PA_ERR_SHAPE;
    *num_waves = w;
    *chunk_fixed = (int32_t)per;
  }
  return PA_OK;
}

// seq_heads > 1: `cache` describes one KV head per block and sequence s
// reads head s % seq_heads of a cache that really holds seq_heads heads per
// block (per-(sequence, head) block tables, as the query-aware decode uses).
pa_status decode(const pa_cache_desc* cache, const void* q, int32_t num_seqs, int32_t num_q_heads,
                 const void* k_cache, const void* v_cache, const int32_t* block_tables,
                 int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t window, float scale,
                 float k_scale, float v_scale, bool fp8, float* out, int32_t partition_tokens,
                 void* workspace, size_t workspace_bytes, void* stream, int32_t seq_heads = 0,
                 float* lse = nullptr, bool append = false, const void* k_new = nullptr,
                 const void* v_new = nullptr, bool ring = false, int32_t unit_charge = -1) {
  if (!cache) return PA_ERR_NULL;
  if (!isfinite(scale) || window < 0) return PA_ERR_SHAPE;
  // Ring rows must hold every block a window can span: ceil(W / BS) + 1.
  if (ring && (window < 1 || cache->block_size < 1 ||
               (int64_t)max_blocks_per_seq < ((int64_t)window + cache->block_size - 1) / cache->block_size + 1))
    return PA_ERR_SHAPE;
  if (fp8 && (!good_scale(k_scale) || !good_scale(v_scale))) return PA_ERR_SHAPE;
  int64_t num_waves = 0;
  int32_t chunk_fixed = 0;
  // Shape checks that need no device come first.
  {
    pa_status st = desc_status(cache);
    if (st != PA_OK) return st;
    if (num_seqs < 0 || num_q_heads < 1 || max_blocks_per_seq < 0) return PA_ERR_SHAPE;
    if (num_q_heads % cache->num_kv_heads != 0) return PA_ERR_SHAPE;
    if (num_q_heads / cache->num_kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
    if (partition_tokens < 0 || partition_tokens % pa::kSub != 0) return PA_ERR_SHAPE;
  }
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out) return PA_ERR_NULL;
  if (append && (!k_new || !v_new)) return PA_ERR_NULL;
  if (!workspace) return PA_ERR_WORKSPACE;
  pa_status st = plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, fp8,
                      &num_waves, &chunk_fixed, window);
  if (st != PA_OK) return st;
  const int group = num_q_heads / cache->num_kv_heads;
  const pa::WorkspaceLayout lay =
      pa::workspace_layout(num_waves, group, cache->head_dim, num_seqs, cache->num_kv_heads);
  if (workspace_bytes < lay.total) return PA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  pa::DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const uint8_t*>(k_cache);
  p.v_cache = static_cast<const uint8_t*>(v_cache);
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.out = out;
  p.lse = lse;
  p.partials = reinterpret_cast<float*>(ws + lay.partials_off);
  p.counters = reinterpret_cast<int32_t*>(ws + lay.counters_off);
  // The merge tree counts groups of pieces by record slot (2 per wavefront).
  p.group_counters = 2 * num_waves <= pa::kGroupCounters
                         ? reinterpret_cast<int32_t*>(ws + lay.group_counters_off)
                         : nullptr;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = cache->num_kv_heads;
  p.group = group;
  p.head_dim = cache->head_dim;
  p.block_size = cache->block_size;
  p.num_blocks = cache->num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.num_waves = (int32_t)num_waves;
  p.chunk_min = kChunkMinAuto;
  p.chunk_fixed = chunk_fixed;
  // unit_charge < 0: the dtype's default.
  p.unit_charge = chunk_fixed > 0         ? 0
                  : unit_charge >= 0      ? unit_charge
                  : fp8                   ? PA_DECODE_UNIT_CHARGE_FP8
                                          : PA_DECODE_UNIT_CHARGE;
  p.window = window;
  p.ring = ring ? 1 : 0;
  p.subs = cache->block_size / pa::kSub;
  p.subs_magic = p.subs > 1 ? (uint32_t)((((uint64_t)1 << 32) + p.subs - 1) / p.subs) : 0u;
  const int32_t heads_per_block = seq_heads > 1 ? seq_heads : cache->num_kv_heads;
  p.blk_stride = (int64_t)heads_per_block * p.subs * pa::kSub * cache->head_dim * (fp8 ? 1 : 2);
  p.seq_heads = seq_heads > 1 ? seq_heads : 0;
  p.seq_heads_magic = seq_heads > 1 ? (uint32_t)((((uint64_t)1 << 32) + seq_heads - 1) / seq_heads) : 0u;
  p.qk_scale = scale * 1.4426950408889634f * (fp8 ? k_scale : 1.0f);
  p.out_scale = fp8 ? v_scale : 1.0f;
  // Fused append: the caches are the caller's writable memory.
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.k_store = append ? const_cast<uint8_t*>(p.k_cache) : nullptr;
  p.v_store = append ? const_cast<uint8_t*>(p.v_cache) : nullptr;
  // The cache write's reciprocals: correctly rounded float32 (IEEE division).
  volatile float one = 1.0f;
  p.k_inv = fp8 ? one / k_scale : 1.0f;
  p.v_inv = fp8 ? one / v_scale : 1.0f;
  if (pa::launch_decode(p, fp8, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

// Shared checks of the block copy / swap entry points: block bytes of the
// cache layout, and a launch grid (items * 2 caches * 16 KiB segments) that
// fits.
pa_status block_move_check(const pa_cache_desc* cache, int32_t elem_bytes, int32_t n,
                           int64_t* block_bytes) {
  if (!cache) return PA_ERR_NULL;
  pa_status st = desc_status(cache);
  if (st != PA_OK) return st;
  if (elem_bytes != 1 && elem_bytes != 2) return PA_ERR_UNSUPPORTED;
  if (n < 0) return PA_ERR_SHAPE;
  *block_bytes = (int64_t)cache->num_kv_heads * cache->block_size * cache->head_dim * elem_bytes;
  if ((int64_t)n * 2 * ((*block_bytes + 16383) / 16384) > INT32_MAX) return PA_ERR_SHAPE;
  return PA_OK;
}

// The device address of pinned host memory (hipHostMalloc); false for any
// other pointer.  The failed query's error is cleared so that it is not
// reported by a later launch check.
bool host_mapping(const void* host, uint8_t** mapped) {
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<void*>(host), 0) != hipSuccess || !d) {
    (void)hipGetLastError();
    return false;
  }
  *mapped = static_cast<uint8_t*>(d);
  return true;
}

pa::BlockMoveParams block_move_params(int64_t block_bytes, int32_t n) {
  pa::BlockMoveParams p{};
  p.block_bytes = block_bytes;
  p.segs = (int32_t)((block_bytes + 16383) / 16384);
  p.last_words = (int32_t)((block_bytes - (int64_t)(p.segs - 1) * 16384) / 16);
  p.num_items = n;
  return p;
}

}  // namespace

// Device scratch of pa_decode_noalloc: the decode workspace of callers that
// cannot allocate (merge counters first, then the partial records).  Each
// device the library runs on holds its own copy, until the process ends.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

void* g_scratch[kMaxDevices];  // per device: the device address of `scratch`

// The device address of this device's copy of `scratch`, looked up once per
// device with that device current (the array's name is a host-side stand-in,
// not a device address).  Null on failure.
void* noalloc_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

pa_status pa_cache_write(const pa_cache_desc* cache, const void* k, const void* v,
                         const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                         void* v_cache, void* stream) {
  return cache_write(cache, k, v, slot_mapping, num_tokens, k_cache, v_cache, false, 1.f, 1.f,
                     stream);
}

pa_status pa_cache_write_fp8(const pa_cache_desc* cache, const void* k, const void* v,
                             const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                             void* v_cache, float k_scale, float v_scale, void* stream) {
  return cache_write(cache, k, v, slot_mapping, num_tokens, k_cache, v_cache, true, k_scale,
                     v_scale, stream);
}

size_t pa_decode_workspace_size(const pa_cache_desc* cache, int32_t num_seqs, int32_t num_q_heads,
                                int32_t max_blocks_per_seq, int32_t partition_tokens) {
  int64_t w16 = 0, w8 = 0;
  int32_t cf = 0;
  if (plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, false, &w16, &cf) !=
      PA_OK)
    return 0;
  if (plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, true, &w8, &cf) !=
      PA_OK)
    return 0;
  const int group = num_q_heads / cache->num_kv_heads;
  const pa::WorkspaceLayout lay = pa::workspace_layout(w16 > w8 ? w16 : w8, group, cache->head_dim,
                                                       num_seqs, cache->num_kv_heads);
  return lay.total;
}

pa_status pa_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return PA_OK;
  if (!workspace) return PA_ERR_NULL;
  int resident = 0;
  if (!device_info(128, false, &resident)) return PA_ERR_DEVICE;
  if (pa::launch_zero(workspace, workspace_bytes, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_decode(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                    int32_t num_q_heads, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, float scale, float* out, int32_t partition_tokens,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode(cache, q, num_seqs, num_q_heads, k_cache, v_cache, block_tables,
                max_blocks_per_seq, seq_lens, 0, scale, 1.f, 1.f, false, out, partition_tokens,
                workspace, workspace_bytes, stream);
}

pa_status pa_decode_noalloc(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                            int32_t num_q_heads, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, float scale, float* out,
                            int32_t partition_tokens, void* stream) {
  // Every check pa_decode makes comes before anything is launched.
  if (!cache) return PA_ERR_NULL;
  if (!isfinite(scale)) return PA_ERR_SHAPE;
  int64_t num_waves = 0;
  int32_t chunk_fixed = 0;
  {
    pa_status st = desc_status(cache);
    if (st != PA_OK) return st;
    if (num_seqs < 0 || num_q_heads < 1 || max_blocks_per_seq < 0) return PA_ERR_SHAPE;
    if (num_q_heads % cache->num_kv_heads != 0) return PA_ERR_SHAPE;
    if (num_q_heads / cache->num_kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
    if (partition_tokens < 0 || partition_tokens % pa::kSub != 0) return PA_ERR_SHAPE;
  }
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out) return PA_ERR_NULL;
  pa_status st = plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, false,
                      &num_waves, &chunk_fixed);
  if (st != PA_OK) return st;
  const pa::WorkspaceLayout lay = pa::workspace_layout(num_waves, num_q_heads / cache->num_kv_heads,
                                                       cache->head_dim, num_seqs, cache->num_kv_heads);
  if (lay.total > kNoAllocScratchBytes) return PA_ERR_WORKSPACE;
  void* ws = noalloc_scratch();
  if (!ws) return PA_ERR_DEVICE;
  // The array keeps the previous call's contents: clear the merge counters
  // (a fill kernel on the caller's stream, ahead of the decode).
  if (pa::launch_zero(ws, lay.partials_off, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return decode(cache, q, num_seqs, num_q_heads, k_cache, v_cache, block_tables, max_blocks_per_seq,
                seq_lens, 0, scale, 1.f, 1.f, false, out, partition_tokens, ws, kNoAllocScratchBytes,
                stream);
}

pa_status pa_decode_window(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                           int32_t num_q_heads, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t window, float scale, float* out,
                           int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return decode(cache, q, num_seqs, num_q_heads, k_cache, v_cache, block_tables,
                max_blocks_per_seq, seq_lens, window, scale, 1.f, 1.f, false, out,
                partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_decode_fp8(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                        int32_t num_q_heads, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* seq_lens, float scale, float k_scale, float v_scale,
                        float* out, int32_t partition_tokens, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return decode(cache, q, num_seqs, num_q_heads, k_cache, v_cache, block_tables,
                max_blocks_per_seq, seq_lens, 0, scale, k_scale, v_scale, true, out,
                partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_decode_window_fp8(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                               int32_t num_q_heads, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, int32_t window, float scale,
                               float k_scale, float v_scale, float* out, int32_t partition_tokens,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return decode(cache, q, num_seqs, num_q_heads, k_cache, v_cache, block_tables,
                max_blocks_per_seq, seq_lens, window, scale, k_scale, v_scale, true, out,
                partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_decode_append(const pa_cache_desc* cache, const void* q, const void* k_new,
                           const void* v_new, int32_t num_seqs, int32_t num_q_heads, void* k_cache,
                           void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t window, float scale, float* out,
                           int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return decode(cache, q, num_seqs, num_q_heads, k_cache, v_cache, block_tables,
                max_blocks_per_seq, seq_lens, window, scale, 1.f, 1.f, false, out,
                partition_tokens, workspace, workspace_bytes, stream, 0, nullptr, true, k_new,
                v_new);
}

pa_status pa_decode_append_fp8(const pa_cache_desc* cache, const void* q, const void* k_new,
                               const void* v_new, int32_t num_seqs, int32_t num_q_heads,
                               void* k_cache, void* v_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t window,
                               float scale, float k_scale, float v_scale, float* out,
                               int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return decode(cache, q, num_seqs, num_q_heads, k_cache, v_cache, block_tables,
                max_blocks_per_seq, seq_lens, window, scale, k_scale, v_scale, true, out,
                partition_tokens, workspace, workspace_bytes, stream, 0, nullptr, true, k_new,
                v_new);
}

pa_status pa_decode_ring(const pa_cache_desc* cache, const void* q, const void* k_new,
                         const void* v_new, int32_t num_seqs, int32_t num_q_heads, void* k_cache,
                         void* v_cache, const int32_t* ring_tables, int32_t ring_entries,
                         const int32_t* seq_lens, int32_t window, float scale, float* out,
                         int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_NULL;
  return decode(cache, q, num_seqs, num_q_heads, k_cache, v_cache, ring_tables, ring_entries,
                seq_lens, window, scale, 1.f, 1.f, false, out, partition_tokens, workspace,
                workspace_bytes, stream, 0, nullptr, k_new != nullptr, k_new, v_new, true);
}

pa_status pa_decode_ring_fp8(const pa_cache_desc* cache, const void* q, const void* k_new,
                             const void* v_new, int32_t num_seqs, int32_t num_q_heads,
                             void* k_cache, void* v_cache, const int32_t* ring_tables,
                             int32_t ring_entries, const int32_t* seq_lens, int32_t window,
                             float scale, float k_scale, float v_scale, float* out,
                             int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_NULL;
  return decode(cache, q, num_seqs, num_q_heads, k_cache, v_cache, ring_tables, ring_entries,
                seq_lens, window, scale, k_scale, v_scale, true, out, partition_tokens, workspace,
                workspace_bytes, stream, 0, nullptr, k_new != nullptr, k_new, v_new, true);
}

pa_status pa_copy_blocks(const pa_cache_desc* cache, int32_t elem_bytes, void* k_cache,
                         void* v_cache, const int32_t* pairs, int32_t num_pairs, void* stream) {
  int64_t block_bytes = 0;
  pa_status st = block_move_check(cache, elem_bytes, num_pairs, &block_bytes);
  if (st != PA_OK || num_pairs == 0) return st;
  if (!k_cache || !v_cache || !pairs) return PA_ERR_NULL;
  int resident = 0;
  if (!device_info(128, false, &resident)) return PA_ERR_DEVICE;
  pa::BlockMoveParams p = block_move_params(block_bytes, num_pairs);
  p.src_k = p.dst_k = static_cast<uint8_t*>(k_cache);
  p.src_v = p.dst_v = static_cast<uint8_t*>(v_cache);
  p.src_ids = pairs;
  p.dst_ids = pairs + 1;
  p.id_stride = 2;
  p.src_blocks = p.dst_blocks = cache->num_blocks;
  if (pa::launch_move_blocks(p, 0, static_cast<hipStream_t>(stream)) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_swap_out(const pa_cache_desc* cache, int32_t elem_bytes, const void* k_cache,
                      const void* v_cache, const int32_t* blocks, int32_t num_blocks, void* host,
                      void* stream) {
  int64_t block_bytes = 0;
  pa_status st = block_move_check(cache, elem_bytes, num_blocks, &block_bytes);
  if (st != PA_OK || num_blocks == 0) return st;
  if (!k_cache || !v_cache || !blocks || !host) return PA_ERR_NULL;
  int resident = 0;
  if (!device_info(128, false, &resident)) return PA_ERR_DEVICE;
  uint8_t* mapped = nullptr;
  if (!host_mapping(host, &mapped)) return PA_ERR_HOST_MEMORY;
  pa::BlockMoveParams p = block_move_params(block_bytes, num_blocks);
  p.src_k = static_cast<const uint8_t*>(k_cache);
  p.src_v = static_cast<const uint8_t*>(v_cache);
  p.dst_k = mapped;
  p.dst_v = mapped + (size_t)num_blocks * block_bytes;
  p.src_ids = blocks;
  p.id_stride = 1;
  p.src_blocks = cache->num_blocks;
  p.dst_blocks = num_blocks;
  if (pa::launch_move_blocks(p, PA_SWAP_GROUPS, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_swap_in(const pa_cache_desc* cache, int32_t elem_bytes, void* k_cache, void* v_cache,
                     const int32_t* blocks, int32_t num_blocks, const void* host, void* stream) {
  int64_t block_bytes = 0;
  pa_status st = block_move_check(cache, elem_bytes, num_blocks, &block_bytes);
  if (st != PA_OK || num_blocks == 0) return st;
  if (!k_cache || !v_cache || !blocks || !host) return PA_ERR_NULL;
  int resident = 0;
  if (!device_info(128, false, &resident)) return PA_ERR_DEVICE;
  uint8_t* mapped = nullptr;
  if (!host_mapping(host, &mapped)) return PA_ERR_HOST_MEMORY;
  pa::BlockMoveParams p = block_move_params(block_bytes, num_blocks);
  p.src_k = mapped;
  p.src_v = mapped + (size_t)num_blocks * block_bytes;
  p.dst_k = static_cast<uint8_t*>(k_cache);
  p.dst_v = static_cast<uint8_t*>(v_cache);
  p.dst_ids = blocks;
  p.id_stride = 1;
  p.src_blocks = num_blocks;
  p.dst_blocks = cache->num_blocks;
  if (pa::launch_move_blocks(p, PA_SWAP_GROUPS, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_quest_clear(const pa_cache_desc* cache, uint32_t* summaries, void* stream) {
  if (!cache) return PA_ERR_NULL;
  pa_status st = desc_status(cache);
  if (st != PA_OK) return st;
  if (!summaries) return PA_ERR_NULL;
  int resident = 0;
  if (!device_info(128, false, &resident)) return PA_ERR_DEVICE;
  const int64_t words = (int64_t)cache->num_blocks * cache->num_kv_heads * cache->head_dim;
  if (pa::launch_summary_fill(summaries, words, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

namespace {

// Shared checks of the summary entry points; fills the common parameters.
pa_status summary_params(const pa_cache_desc* cache, int32_t elem_bytes, const void* k_cache,
                         int32_t n, uint32_t* summaries, pa::SummaryParams* p) {
  if (!cache) return PA_ERR_NULL;
  pa_status st = desc_status(cache);
  if (st != PA_OK) return st;
  if (elem_bytes != 1 && elem_bytes != 2) return PA_ERR_UNSUPPORTED;
  if (n < 0) return PA_ERR_SHAPE;
  // Threads of the largest launch: n * Hkv * (D / 4) must fit the grid.
  if ((int64_t)n * cache->num_kv_heads * (cache->head_dim / 4) > (int64_t)INT32_MAX * 128)
    return PA_ERR_SHAPE;
  if (n > 0 && (!k_cache || !summaries)) return PA_ERR_NULL;
  *p = pa::SummaryParams{};
  p->k_cache = static_cast<const uint8_t*>(k_cache);
  p->words = summaries;
  p->num_tokens = n;
  p->num_kv_heads = cache->num_kv_heads;
  p->head_dim = cache->head_dim;
  p->block_size = cache->block_size;
  p->num_blocks = cache->num_blocks;
  return PA_OK;
}

}  // namespace

pa_status pa_quest_cache_write(const pa_cache_desc* cache, const void* k, const void* v,
                               const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                               void* v_cache, uint32_t* summaries, void* stream) {
  if (num_tokens > 0 && !summaries) return PA_ERR_NULL;
  return cache_write(cache, k, v, slot_mapping, num_tokens, k_cache, v_cache, false, 1.f, 1.f, stream,
                     summaries);
}

pa_status pa_quest_cache_write_fp8(const pa_cache_desc* cache, const void* k, const void* v,
                                   const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                                   void* v_cache, float k_scale, float v_scale, uint32_t* summaries,
                                   void* stream) {
  if (num_tokens > 0 && !summaries) return PA_ERR_NULL;
  return cache_write(cache, k, v, slot_mapping, num_tokens, k_cache, v_cache, true, k_scale, v_scale, stream,
                     summaries);
}

pa_status pa_quest_update(const pa_cache_desc* cache, int32_t elem_bytes, const void* k_cache,
                          const int64_t* slot_mapping, int32_t num_tokens, uint32_t* summaries,
                          void* stream) {
  pa::SummaryParams p;
  pa_status st = summary_params(cache, elem_bytes, k_cache, num_tokens, summaries, &p);
  if (st != PA_OK || num_tokens == 0) return st;
  if (!slot_mapping) return PA_ERR_NULL;
  int resident = 0;
  if (!device_info(128, false, &resident)) return PA_ERR_DEVICE;
  p.slots = slot_mapping;
  if (pa::launch_summary_update(p, elem_bytes == 1, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_quest_summarize(const pa_cache_desc* cache, int32_t elem_bytes, const void* k_cache,
                             const int32_t* blocks, const int32_t* counts, int32_t num_items,
                             uint32_t* summaries, void* stream) {
  pa::SummaryParams p;
  pa_status st = summary_params(cache, elem_bytes, k_cache, num_items, summaries, &p);
  if (st != PA_OK || num_items == 0) return st;
  if (!blocks || !counts) return PA_ERR_NULL;
  int resident = 0;
  if (!device_info(128, false, &resident)) return PA_ERR_DEVICE;
  p.blocks = blocks;
  p.counts = counts;
  if (pa::launch_summary_build(p, elem_bytes == 1, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

size_t pa_quest_select_workspace_size(int32_t num_seqs, int32_t num_kv_heads,
                                      int32_t max_blocks_per_seq) {
  if (num_seqs < 0 || num_kv_heads < 1 || max_blocks_per_seq < 0) return 0;
  return pa::align_up((size_t)num_seqs * num_kv_heads * (size_t)max_blocks_per_seq * sizeof(uint32_t),
                      256);
}

pa_status pa_quest_select(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                          int32_t num_q_heads, const uint32_t* summaries,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, int32_t budget, int32_t* sel_tables,
                          int32_t* sel_lens, void* workspace, size_t workspace_bytes, void* stream) {
  if (!cache) return PA_ERR_NULL;
  pa_status st = desc_status(cache);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads < 1 || max_blocks_per_seq < 0 || budget < 1) return PA_ERR_SHAPE;
  if (num_q_heads % cache->num_kv_heads != 0) return PA_ERR_SHAPE;
  if (num_q_heads / cache->num_kv_heads > pa::kMaxGroupQuest) return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_blocks_per_seq * cache->block_size > INT32_MAX) return PA_ERR_SHAPE;
  const int64_t units = (int64_t)num_seqs * cache->num_kv_heads;
  if (units * (int64_t)(max_blocks_per_seq > 0 ? max_blocks_per_seq : 1) > INT32_MAX ||
      units * budget > INT32_MAX)
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!q || !summaries || !block_tables || !seq_lens || !sel_tables || !sel_lens) return PA_ERR_NULL;
  const size_t need = pa_quest_select_workspace_size(num_seqs, cache->num_kv_heads, max_blocks_per_seq);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  int resident = 0;
  if (!device_info(cache->head_dim, false, &resident)) return PA_ERR_DEVICE;
  pa::SelectParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.words = summaries;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.keys = static_cast<uint32_t*>(workspace);
  p.sel_tables = sel_tables;
  p.sel_lens = sel_lens;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = cache->num_kv_heads;
  p.group = num_q_heads / cache->num_kv_heads;
  p.head_dim = cache->head_dim;
  p.block_size = cache->block_size;
  p.num_blocks = cache->num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.budget = budget;
  if (pa::launch_page_select(p, static_cast<hipStream_t>(stream)) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

namespace {

// The cache as the decode over per-(sequence, head) tables sees it: one KV
// head per block, the sequences being (s, h) pairs.
pa_status quest_view(const pa_cache_desc* cache, int32_t num_seqs, int32_t num_q_heads,
                     pa_cache_desc* view, int32_t* units, int32_t* group) {
  if (!cache) return PA_ERR_NULL;
  pa_status st = desc_status(cache);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads < 1 || num_q_heads % cache->num_kv_heads != 0) return PA_ERR_SHAPE;
  if ((int64_t)num_seqs * cache->num_kv_heads > INT32_MAX) return PA_ERR_SHAPE;
  *view = *cache;
  view->num_kv_heads = 1;
  *units = num_seqs * cache->num_kv_heads;
  *group = num_q_heads / cache->num_kv_heads;
  return PA_OK;
}

pa_status decode_quest(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                       int32_t num_q_heads, const void* k_cache, const void* v_cache,
                       const int32_t* sel_tables, int32_t budget, const int32_t* sel_lens,
                       float scale, float k_scale, float v_scale, bool fp8, float* out,
                       int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                       void* stream) {
  pa_cache_desc view;
  int32_t units = 0, group = 0;
  pa_status st = quest_view(cache, num_seqs, num_q_heads, &view, &units, &group);
  if (st != PA_OK) return st;
  if (budget < 1) return PA_ERR_SHAPE;
  // q [S][Hq][D] is [S * Hkv][G][D], and so is out.
  return decode(&view, q, units, group, k_cache, v_cache, sel_tables, budget, sel_lens, 0, scale,
                k_scale, v_scale, fp8, out, partition_tokens, workspace, workspace_bytes, stream,
                cache->num_kv_heads);
}

}  // namespace

size_t pa_decode_quest_workspace_size(const pa_cache_desc* cache, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t budget,
                                      int32_t partition_tokens) {
  pa_cache_desc view;
  int32_t units = 0, group = 0;
  if (quest_view(cache, num_seqs, num_q_heads, &view, &units, &group) != PA_OK || budget < 1) return 0;
  return pa_decode_workspace_size(&view, units, group, budget, partition_tokens);
}

pa_status pa_decode_quest(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                          int32_t num_q_heads, const void* k_cache, const void* v_cache,
                          const int32_t* sel_tables, int32_t budget, const int32_t* sel_lens,
                          float scale, float* out, int32_t partition_tokens, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return decode_quest(cache, q, num_seqs, num_q_heads, k_cache, v_cache, sel_tables, budget, sel_lens,
                      scale, 1.f, 1.f, false, out, partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_decode_quest_fp8(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                              int32_t num_q_heads, const void* k_cache, const void* v_cache,
                              const int32_t* sel_tables, int32_t budget, const int32_t* sel_lens,
                              float scale, float k_scale, float v_scale, float* out,
                              int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return decode_quest(cache, q, num_seqs, num_q_heads, k_cache, v_cache, sel_tables, budget, sel_lens,
                      scale, k_scale, v_scale, true, out, partition_tokens, workspace, workspace_bytes,
                      stream);
}

namespace {

// Workspace of the cascade decode: the private decode's workspace first (so
// a zero fill of the whole buffer arms its counters), then the private
// outputs and log-sum-exps, then the partial records.
struct CascadeLayout {
  size_t dec_bytes, out_off, lse_off, part_off, total;
};

bool cascade_layout(const pa_cache_desc* cache, int32_t S, int32_t Hq, int32_t maxb, int32_t slots,
                    int32_t partition_tokens, CascadeLayout* lay) {
  if (slots < 0) return false;
  const size_t dec = pa_decode_workspace_size(cache, S, Hq, maxb, partition_tokens);
  if (dec == 0 && S > 0) return false;
  const size_t D = cache->head_dim;
  lay->dec_bytes = dec;
  lay->out_off = pa::align_up(dec, 256);
  lay->lse_off = pa::align_up(lay->out_off + (size_t)S * Hq * D * sizeof(float), 256);
  lay->part_off = pa::align_up(lay->lse_off + (size_t)S * Hq * sizeof(float), 256);
  lay->total = pa::align_up(lay->part_off + (size_t)slots * Hq * (D + 4) * sizeof(float), 256);
  return true;
}

pa_status decode_cascade(const pa_cache_desc* cache, const void* q, int32_t S, int32_t Hq,
                         const void* k_cache, const void* v_cache, int32_t maxb,
                         const pa_cascade_device_plan* plan, float scale, float k_scale, float v_scale,
                         bool fp8, float* out, int32_t partition_tokens, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!cache || !plan) return PA_ERR_NULL;
  pa_status st = desc_status(cache);
  if (st != PA_OK) return st;
  if (S < 0 || Hq < 1 || maxb < 0 || Hq % cache->num_kv_heads != 0) return PA_ERR_SHAPE;
  const int32_t G = Hq / cache->num_kv_heads;
  if (G > 16) return PA_ERR_UNSUPPORTED;
  if (!isfinite(scale) || plan->num_items < 0 || plan->num_slots < 0) return PA_ERR_SHAPE;
  if (fp8 && (!good_scale(k_scale) || !good_scale(v_scale))) return PA_ERR_SHAPE;
  if (S == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !out || !plan->parts_off || !plan->private_tables ||
      !plan->private_lens || (plan->num_items > 0 && (!plan->items || !plan->seg_blocks || !plan->members)) ||
      (plan->num_slots > 0 && !plan->parts))
    return PA_ERR_NULL;
  int resident = 0;
  if (!device_info(cache->head_dim, fp8, &resident)) return PA_ERR_DEVICE;
  CascadeLayout lay;
  if (!cascade_layout(cache, S, Hq, maxb, plan->num_slots, partition_tokens, &lay)) return PA_ERR_SHAPE;
  if (!workspace || workspace_bytes < lay.total) return PA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* part_out = reinterpret_cast<float*>(ws + lay.out_off);
  float* part_lse = reinterpret_cast<float*>(ws + lay.lse_off);
  float* partials = reinterpret_cast<float*>(ws + lay.part_off);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Private parts (and the device checks) through the paged decode.
  st = decode(cache, q, S, Hq, k_cache, v_cache, plan->private_tables, maxb, plan->private_lens, 0, scale,
              k_scale, v_scale, fp8, part_out, partition_tokens, ws, lay.dec_bytes, stream, 0, part_lse, false,
              nullptr, nullptr, false, fp8 ? -1 : PA_CASCADE_UNIT_CHARGE);
  if (st != PA_OK) return st;
  pa::SegmentParams sp{};
  sp.q = static_cast<const uint16_t*>(q);
  sp.k_cache = static_cast<const uint8_t*>(k_cache);
  sp.v_cache = static_cast<const uint8_t*>(v_cache);
  sp.items = plan->items;
  sp.seg_blocks = plan->seg_blocks;
  sp.members = plan->members;
  sp.partials = partials;
  sp.num_items = plan->num_items;
  sp.num_q_heads = Hq;
  sp.group = G;
  sp.mpw = 16 / G;
  sp.head_dim = cache->head_dim;
  sp.block_size = cache->block_size;
  sp.num_blocks = cache->num_blocks;
  sp.num_seqs = S;
  sp.num_slots = plan->num_slots;
  sp.blk_stride = (int64_t)cache->num_kv_heads * cache->block_size * cache->head_dim * (fp8 ? 1 : 2);
  // scale (q . k) = |scale| ((-q) . k) for scale < 0, exactly: the kernel
  // takes the maximum of its raw logits, which needs a non-negative scale.
  sp.qk_scale = fabsf(scale) * 1.4426950408889634f * (fp8 ? k_scale : 1.0f);
  sp.q_sign = scale < 0.f ? 0x80008000u : 0u;
  if (pa::launch_segments(sp, fp8, s) != hipSuccess) return PA_ERR_LAUNCH;
  pa::CombineParams cp{};
  cp.part_out = part_out;
  cp.part_lse = part_lse;
  cp.partials = partials;
  cp.parts_off = plan->parts_off;
  cp.parts = plan->parts;
  cp.out = out;
  cp.num_seqs = S;
  cp.num_q_heads = Hq;
  cp.head_dim = cache->head_dim;
  cp.num_slots = plan->num_slots;
  cp.out_scale = fp8 ? v_scale : 1.0f;
  if (pa::launch_combine(cp, s) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

}  // namespace

size_t pa_decode_cascade_workspace_size(const pa_cache_desc* cache, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t max_blocks_per_seq, int32_t num_slots,
                                        int32_t partition_tokens) {
  if (!cache || desc_status(cache) != PA_OK) return 0;
  CascadeLayout lay;
  if (!cascade_layout(cache, num_seqs, num_q_heads, max_blocks_per_seq, num_slots, partition_tokens, &lay))
    return 0;
  return lay.total;
}

pa_status pa_decode_cascade(const pa_cache_desc* cache, const void* q, int32_t num_seqs, int32_t num_q_heads,
                            const void* k_cache, const void* v_cache, int32_t max_blocks_per_seq,
                            const pa_cascade_device_plan* plan, float scale, float* out,
                            int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_cascade(cache, q, num_seqs, num_q_heads, k_cache, v_cache, max_blocks_per_seq, plan, scale,
                        1.f, 1.f, false, out, partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_decode_cascade_fp8(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                                int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                int32_t max_blocks_per_seq, const pa_cascade_device_plan* plan, float scale,
                                float k_scale, float v_scale, float* out, int32_t partition_tokens,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return decode_cascade(cache, q, num_seqs, num_q_heads, k_cache, v_cache, max_blocks_per_seq, plan, scale,
                        k_scale, v_scale, true, out, partition_tokens, workspace, workspace_bytes, stream);
}

namespace {

// Workgroups of a probe: 4 per CU of the current device (16 wavefronts).
int probe_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return 4 * cus;
}

}  // namespace

pa_status pa_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!sink || (bytes > 0 && !buf)) return PA_ERR_NULL;
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0) return PA_ERR_SHAPE;
  int resident = 0;
  if (!device_info(128, false, &resident)) return PA_ERR_DEVICE;
  if (bytes == 0) return PA_OK;
  const int grid = probe_grid();
  if (grid <= 0) return PA_ERR_DEVICE;
  if (pa::launch_stream_read(buf, bytes, sink, grid, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_probe_tile_read(const pa_cache_desc* cache, int32_t elem_bytes, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables, int32_t num_seqs,
                             int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t window,
                             uint32_t* sink, void* stream) {
  if (!cache) return PA_ERR_NULL;
  pa_status st = desc_status(cache);
  if (st != PA_OK) return st;
  if (elem_bytes != 1 && elem_bytes != 2) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_blocks_per_seq < 0 || window < 0) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * cache->block_size > INT32_MAX) return PA_ERR_SHAPE;
  if ((int64_t)num_seqs * cache->num_kv_heads * max_blocks_per_seq > INT32_MAX) return PA_ERR_SHAPE;
  if (!sink) return PA_ERR_NULL;
  if (num_seqs == 0 || max_blocks_per_seq == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_tables || !seq_lens) return PA_ERR_NULL;
  int resident = 0;
  if (!device_info(cache->head_dim, elem_bytes == 1, &resident)) return PA_ERR_DEVICE;
  const int grid = probe_grid();
  if (grid <= 0) return PA_ERR_DEVICE;
  pa::TileProbeParams p{};
  p.k_cache = static_cast<const uint8_t*>(k_cache);
  p.v_cache = static_cast<const uint8_t*>(v_cache);
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.sink = sink;
  p.num_seqs = num_seqs;
  p.num_kv_heads = cache->num_kv_heads;
  p.max_blocks = max_blocks_per_seq;
  p.block_size = cache->block_size;
  p.num_blocks = cache->num_blocks;
  p.head_dim = cache->head_dim;
  p.elem_bytes = elem_bytes;
  p.window = window;
  p.blk_stride = (int64_t)cache->num_kv_heads * cache->block_size * cache->head_dim * elem_bytes;
  if (pa::launch_tile_read(p, grid, static_cast<hipStream_t>(stream)) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: sizes inconsistent or out of range";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: head_dim, block_size or group size not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: the HIP runtime reported an error";
    case PA_ERR_DEVICE: return "PA_ERR_DEVICE: no gfx950 device is current";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: not enough free blocks";
    case PA_ERR_NOT_FOUND: return "PA_ERR_NOT_FOUND: unknown or already used sequence id";
    case PA_ERR_SWAPPED: return "PA_ERR_SWAPPED: the sequence is swapped out (or not swapped out)";
    case PA_ERR_HOST_MEMORY: return "PA_ERR_HOST_MEMORY: the host buffer is not pinned (hipHostMalloc) memory";
  }
  return "unknown pa_status";
}

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

}  // extern "C"
