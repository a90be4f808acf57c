// Read-bandwidth probes that set the practical ceilings the decode is
// measured against (include/pa_probe.h):
//
// stream_read_kernel: a plain streaming read of one contiguous buffer; each
// wavefront reads its own contiguous range, 16 KB of loads in flight.
//
// tile_read_kernel: the loads of a paged decode and nothing else.  For every
// (sequence, KV head) it reads the K and V tiles (16 tokens each) that cover
// the sequence's tokens (with a window, its last `window` tokens), through
// the block table, in the cache layout the decode kernel reads ("Taming the token torrent", "The Block Table Logic");
// the tiles are split evenly over the wavefronts, 16 KB of loads in flight
// per wavefront.  No arithmetic on the data.
//
// Both fold every 32-bit word they read into an XOR, reduced per wavefront
// and added to *sink with one atomic XOR, so that the loads cannot be
// dropped and a test can check which bytes were read.
#include "pa_internal.h"

namespace pa {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kInFlight = 16384;  // bytes of loads a wavefront keeps in flight

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__device__ __forceinline__ void wave_xor_out(uint32_t x, uint32_t* sink) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0 && x != 0u) atomicXor(sink, x);
}

__device__ __forceinline__ int64_t wave_id() {
  return (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
}

// Wavefront w reads 1 KB rows [w R / W, (w + 1) R / W) of the buffer, R
// rows in all, kInFlight bytes of them at a time; the tail under 1 KB is
// read by the last wavefront.
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* buf, uint64_t words,
                                                                    uint32_t* sink) {
  constexpr int NB = kInFlight / 1024;
  const int lane = threadIdx.x & 63;
  const int64_t W = (int64_t)gridDim.x * (kProbeThreads / 64), w = wave_id();
  const int64_t rows = (int64_t)(words / 64);
  const int64_t r0 = w * rows / W, r1 = (w + 1) * rows / W;
  uint32_t acc = 0;
  for (int64_t r = r0; r < r1; r += NB) {
    u32x4 v[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int64_t rr = r + k < r1 ? r + k : r1 - 1;   // past the range: reloaded, folded once
      v[k] = __builtin_nontemporal_load(buf + rr * 64 + lane);
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) acc ^= r + k < r1 ? fold(v[k]) : 0u;
  }
  if (w == W - 1)
    for (uint64_t i = (uint64_t)rows * 64 + lane; i < words; i += 64) acc ^= fold(buf[i]);
  wave_xor_out(acc, sink);
}

// The decode's tiles, flattened in (sequence, head, tile) order over the
// sequences with 1 <= len <= max_blocks * block_size; wavefront w reads
// tiles [w T / W, (w + 1) T / W) of the T in all, B tiles (K and V) at a
// time.  Each wavefront finds its first sequence by a scan of the lengths.
// Block ids outside the pool read block 0 and are not folded.  Tile t of a
// sequence is its chunk c0 + t, c0 the chunk holding its first attended
// token (0 without a window).
template <int BYTES>
__global__ __launch_bounds__(kProbeThreads) void tile_read_kernel(const TileProbeParams p) {
  constexpr int NL = BYTES / 1024;              // 16-byte loads per lane and tile
  constexpr int B = kInFlight / (2 * BYTES);    // tiles in flight
  const int lane = threadIdx.x & 63;
  const int subs = p.block_size / kSub;
  const int lmax = p.max_blocks * p.block_size;
  auto first_chunk = [&](int L) -> int { return (p.window > 0 && L > p.window) ? (L - p.window) / kSub : 0; };
  auto ntiles = [&](int s) -> int {
    const int L = p.seq_lens[s];
    return (L >= 1 && L <= lmax) ? (L + kSub - 1) / kSub - first_chunk(L) : 0;
  };
  int64_t total = 0;
  for (int s = lane; s < p.num_seqs; s += 64) total += ntiles(s);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) total += __shfl_xor(total, o, 64);
  total *= p.num_kv_heads;
  const int64_t W = (int64_t)gridDim.x * (kProbeThreads / 64), w = wave_id();
  const int64_t i0 = w * total / W, i1 = (w + 1) * total / W;
  uint32_t acc = 0;
  if (i0 < i1) {
    // The sequence holding flattened tile i0, then (head, tile) inside it.
    int s = 0, nt = 0;
    int64_t base = 0;
    for (;; ++s) {
      nt = ntiles(s);
      if (i0 < base + (int64_t)nt * p.num_kv_heads) break;
      base += (int64_t)nt * p.num_kv_heads;
    }
    int h = (int)((i0 - base) / nt), t = (int)((i0 - base) % nt);
    int c0 = first_chunk(p.seq_lens[s]);
    for (int64_t i = i0; i < i1; i += B) {
      u32x4 r[B][2 * NL];
      bool ok[B];
#pragma unroll
      for (int k = 0; k < B; ++k) {
        ok[k] = i + k < i1;
        const int tc = c0 + t;
        const int blk = __builtin_amdgcn_readfirstlane(p.block_tables[(int64_t)s * p.max_blocks + tc / subs]);
        const bool in_pool = (unsigned)blk < (unsigned)p.num_blocks;
        ok[k] = ok[k] && in_pool;
        const int64_t off = (int64_t)(in_pool ? blk : 0) * p.blk_stride + (int64_t)(h * subs + tc % subs) * BYTES;
        const u32x4* kp = reinterpret_cast<const u32x4*>(p.k_cache + off) + lane;
        const u32x4* vp = reinterpret_cast<const u32x4*>(p.v_cache + off) + lane;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          r[k][j] = __builtin_nontemporal_load(kp + 64 * j);
          r[k][NL + j] = __builtin_nontemporal_load(vp + 64 * j);
        }
        // Next tile: along the sequence, then the next head, then the next
        // sequence that has tiles (only while tiles of the range remain).
        if (i + k + 1 < i1 && ++t == nt) {
          t = 0;
          if (++h == p.num_kv_heads) {
            h = 0;
            do nt = ntiles(++s);
            while (nt == 0);
            c0 = first_chunk(p.seq_lens[s]);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < B; ++k) {
        uint32_t x = 0;
#pragma unroll
        for (int j = 0; j < 2 * NL; ++j) x ^= fold(r[k][j]);
        acc ^= ok[k] ? x : 0u;
      }
    }
  }
  wave_xor_out(acc, p.sink);
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int grid, hipStream_t stream) {
  const uint64_t words = bytes / 16;
  if (words == 0) return hipSuccess;
  const uint64_t rows = words / 64;
  // At least one 1 KB row per wavefront, at most `grid` workgroups.
  const uint64_t need = (rows + 3) / 4;
  if (need < (uint64_t)grid) grid = need > 0 ? (int)need : 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(buf), words, sink);
  return hipGetLastError();
}

hipError_t launch_tile_read(const TileProbeParams& p, int grid, hipStream_t stream) {
  const int bytes = kSub * p.head_dim * p.elem_bytes;
  switch (bytes) {
    case 1024: hipLaunchKernelGGL((tile_read_kernel<1024>), dim3((unsigned)grid), dim3(kProbeThreads), 0, stream, p); break;
    case 2048: hipLaunchKernelGGL((tile_read_kernel<2048>), dim3((unsigned)grid), dim3(kProbeThreads), 0, stream, p); break;
    case 4096: hipLaunchKernelGGL((tile_read_kernel<4096>), dim3((unsigned)grid), dim3(kProbeThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
