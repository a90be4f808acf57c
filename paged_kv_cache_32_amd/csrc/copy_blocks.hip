// Whole-block copies inside the K and V caches (the copy-on-write step of
// the block manager: "Taming the token torrent", "Implementing Radix Tree
// Prefix Caching").  A block of the cache layout is one contiguous run of
// Hkv * block_size * head_dim elements, so a copy is a plain streaming copy
// of block_bytes per cache; the kernel is bound by HBM bandwidth (each pair
// reads and writes 2 * block_bytes).  Sources are read with the
// non-temporal hint and destinations written with ordinary stores: on
// MI355X that measured faster than non-temporal or ordinary accesses on both
// sides.
#include "pa_internal.h"

namespace pa {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Workgroup (pair, cache, segment): 256 lanes move one segment of one block
// of one cache, 16 bytes per lane per step.  Every segment is kSegment bytes
// except a block's last, whose 16-byte word count the host computes.
constexpr int kSegment = 16384;
constexpr int kSegWords = kSegment / 16;

__global__ __launch_bounds__(256) void copy_blocks_kernel(const CopyBlocksParams p) {
  const int segs = p.segs;
  const int w = blockIdx.x;
  const int pair = w / (2 * segs);
  const int rest = w - pair * 2 * segs;
  const int cache = rest / segs;
  const int seg = rest - cache * segs;
  const int src = p.pairs[2 * pair], dst = p.pairs[2 * pair + 1];
  if ((unsigned)src >= (unsigned)p.num_blocks || (unsigned)dst >= (unsigned)p.num_blocks) return;
  uint8_t* base = cache ? p.v_cache : p.k_cache;
  const int64_t off = (int64_t)seg * kSegment;
  const u32x4* from = reinterpret_cast<const u32x4*>(base + (int64_t)src * p.block_bytes + off);
  u32x4* to = reinterpret_cast<u32x4*>(base + (int64_t)dst * p.block_bytes + off);
  const int lane = threadIdx.x;
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

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t stream) {
  if (p.num_pairs == 0) return hipSuccess;
  const int64_t groups = (int64_t)p.num_pairs * 2 * p.segs;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)groups), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
