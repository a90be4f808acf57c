// Whole-block moves: copies inside the K and V caches (the copy-on-write step
// of the block manager: "Taming the token torrent", "Implementing Radix Tree
// Prefix Caching"), and swaps of blocks to and from pinned host memory
// ("Taming the token torrent", "The Swapping Mechanism"; "KV Cache
// Engineering for LLM Serving", section 12).  A block of the cache layout is
// one contiguous run of Hkv * block_size * head_dim elements, so a move is a
// plain streaming copy of block_bytes per cache.
//
// In the cache, a copy is bound by HBM bandwidth (each pair reads and writes
// 2 * block_bytes) and runs one workgroup per 16 KiB segment.  A swap reads or
// writes the host buffer directly through its device mapping, bound by the
// host link; it runs on a small, capped grid whose workgroups stride over the
// segments, so a swap beside a decode holds few wave slots and few requests
// in the memory system at once.  Sources are read with the non-temporal hint
// and destinations written with ordinary stores: on MI355X that measured
// faster than non-temporal or ordinary accesses on both sides.
#include "pa_internal.h"

namespace pa {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Work unit (item, cache, segment): 256 lanes move one segment of one block
// of one cache, 16 bytes per lane per step.  Every segment is kSegment bytes
// except a block's last, whose 16-byte word count the host computes.  Item i
// moves source block src_ids[i * id_stride] (or block i when src_ids is
// null) to destination block dst_ids[i * id_stride] (or i); ids outside
// their buffer's block count skip the item.  Workgroup g takes units g,
// g + grid, g + 2 grid, ... (the host keeps the unit count below 2^31).
constexpr int kSegment = 16384;
constexpr int kSegWords = kSegment / 16;

__global__ __launch_bounds__(256) void move_blocks_kernel(const BlockMoveParams p) {
  const unsigned segs = p.segs;
  const unsigned units = (unsigned)p.num_items * 2u * segs;
  const int lane = threadIdx.x;
  for (unsigned w = blockIdx.x; w < units; w += gridDim.x) {
    const unsigned item = w / (2u * segs);
    const unsigned rest = w - item * 2u * segs;
    const unsigned cache = rest / segs;
    const unsigned seg = rest - cache * segs;
    const int src = p.src_ids ? p.src_ids[(int64_t)item * p.id_stride] : (int)item;
    const int dst = p.dst_ids ? p.dst_ids[(int64_t)item * p.id_stride] : (int)item;
    if ((unsigned)src >= (unsigned)p.src_blocks || (unsigned)dst >= (unsigned)p.dst_blocks) continue;
    const int64_t off = (int64_t)seg * kSegment;
    const u32x4* from =
        reinterpret_cast<const u32x4*>((cache ? p.src_v : p.src_k) + (int64_t)src * p.block_bytes + off);
    u32x4* to = reinterpret_cast<u32x4*>((cache ? p.dst_v : p.dst_k) + (int64_t)dst * p.block_bytes + off);
    if (seg + 1 < segs || p.last_words == kSegWords) {
      // Whole segment: all of this lane's loads in flight before any store.
      constexpr int kPer = kSegWords / 256;
      u32x4 r[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) r[i] = __builtin_nontemporal_load(from + lane + 256 * i);
#pragma unroll
      for (int i = 0; i < kPer; ++i) to[lane + 256 * i] = r[i];
    } else {
      for (int i = lane; i < p.last_words; i += 256) to[i] = __builtin_nontemporal_load(from + i);
    }
  }
}

}  // namespace

hipError_t launch_move_blocks(const BlockMoveParams& p, int max_groups, hipStream_t stream) {
  if (p.num_items == 0) return hipSuccess;
  int64_t groups = (int64_t)p.num_items * 2 * p.segs;
  if (max_groups > 0 && groups > max_groups) groups = max_groups;
  hipLaunchKernelGGL(move_blocks_kernel, dim3((unsigned)groups), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
