// Slot scatter of new tokens' K/V into the paged cache (bf16 and fp8).
//
// A slot is a physical token position, block * block_size + offset; the new
// token of a sequence goes to the slot its block table gives for its
// position ("Taming the token torrent", "The Block Table Logic";
// rajatmohan.com serving design, "Paging, because contiguous allocation is
// a disaster").  The fp8 variant stores e4m3fn codes of x / scale, rounded
// to nearest even and saturated ("KV Cache Engineering for LLM Serving",
// section 8, Quantization).
//
// With a summary array (the query-aware page selection of "KV Cache
// Engineering for LLM Serving", section 7), the same threads keep each
// block's per-dimension key minimum and maximum current: a token at offset 0
// starts its block's summary, any other token widens it.  That is a plain
// read-modify-write of the words, valid because no two tokens of one such
// call share a block (the caller's contract: a decode step's new tokens,
// one per sequence, each in a block its sequence owns alone).
//
// A decode step's write is a few hundred bytes per token: it is latency
// bound, so that kernel is one thread per 16-byte K chunk of a (token, kv
// head) row, with the matching V elements.  Bulk writes use a tile kernel
// (below).  A token's K row and V
// column write many cache lines in part (16-byte K pieces 256 bytes apart, V
// elements spread over the whole V tile); the stores carry the non-temporal
// hint so that those lines are not kept in L2 as partly written lines when
// the decode then streams the cache through it.
#include "pa_internal.h"

namespace pa {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Calls with at least this many tokens take the tile kernel.
constexpr int kTileWriteMinTokens = 512;

// bf16 bits of an e4m3fn code's value (no scale): exact; a NaN code gives
// a bf16 NaN.
__device__ __forceinline__ uint32_t e4m3_bf16_bits(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 8;
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  if (e == 15u && m == 7u) return sign | 0x7FC0u;
  if (e == 0u) return sign | (__float_as_uint((float)m * 0x1p-9f) >> 16);
  return sign | ((e + 120u) << 7) | (m << 4);
}

// The summary words of X consecutive key dimensions (dg * X ..) of one
// (block, head): a token at offset 0 sets them from its own key (a NaN key
// leaves a dimension empty), any other token widens them.  `key` holds the
// stored keys' bf16 bits.
template <int X>
__device__ __forceinline__ void update_summary(const CacheWriteParams& p, int64_t blk, int h, int dg, bool first,
                                               const uint32_t (&key)[X]) {
#pragma unroll
  for (int qd = 0; qd < X / 4; ++qd) {
    u32x4* w = reinterpret_cast<u32x4*>(p.summaries + summary_word(blk, h, dg * X + 4 * qd, p.num_kv_heads, p.head_dim));
    u32x4 cur = first ? u32x4{kEmptySummaryWord, kEmptySummaryWord, kEmptySummaryWord, kEmptySummaryWord} : *w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t vb = key[4 * qd + e];
      const float v = bf16_to_f32(vb);
      const uint32_t lo = cur[e] & 0xFFFFu, hi = cur[e] >> 16;
      const uint32_t nlo = v < bf16_to_f32(lo) ? vb : lo;   // a NaN compares false: unchanged
      const uint32_t nhi = v > bf16_to_f32(hi) ? vb : hi;
      cur[e] = (nhi << 16) | nlo;
    }
    *w = cur;
  }
}

// One (token j, kv head h, group dg of X elements) of a row, X = 16 bytes of
// cache: 8 bf16 values or 16 fp8 codes: the K piece, the matching V
// elements and (QUEST) the summary words of those X dimensions.
template <bool FP8, bool QUEST>
__device__ __forceinline__ void write_group(const CacheWriteParams& p, int j, int h, int dg) {
  constexpr int X = FP8 ? 16 : 8;
  const int64_t slot = p.slots[j];
  if (slot < 0 || slot >= p.num_slots) return;
  const int64_t blk = slot / p.block_size;
  const int off = (int)(slot - blk * p.block_size);
  const int sub = off / kSub, r = off % kSub;
  const int subs = p.block_size / kSub;
  // Byte offset of this (block, head, sub-block) tile; K and V tiles have the
  // same size: 16 tokens x head_dim elements.
  const int eb = FP8 ? 1 : 2;
  const int64_t tile = (((blk * p.num_kv_heads + h) * subs + sub) * (int64_t)(kSub * p.head_dim)) * eb;

  const int64_t src = ((int64_t)j * p.num_kv_heads + h) * p.head_dim + (int64_t)dg * X;
  uint8_t* kdst = p.k_cache + tile + ((int64_t)dg * kSub + r) * 16;    // [d/X][t%16][X]
  uint8_t* vtile = p.v_cache + tile;  // [d/16R][d%16][(t%16)/4][(d/16)%R][t%4], R = 4 / eb
  if (!FP8) {
    const u32x4 kv = *reinterpret_cast<const u32x4*>(p.k + src);
    __builtin_nontemporal_store(kv, reinterpret_cast<u32x4*>(kdst));
    if constexpr (QUEST) {
      uint32_t key[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) key[e] = (e & 1) ? (kv[e >> 1] >> 16) : (kv[e >> 1] & 0xFFFFu);
      update_summary<8>(p, blk, h, dg, off == 0, key);
    }
    const u32x4 vv = *reinterpret_cast<const u32x4*>(p.v + src);
    uint16_t* vdst = reinterpret_cast<uint16_t*>(vtile);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = vv[e >> 1];
      __builtin_nontemporal_store((uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu)), vdst + v_elem<2>(dg * 8 + e, r));
    }
  } else {
    u32x4 kin[2], vin[2];
    kin[0] = *reinterpret_cast<const u32x4*>(p.k + src);
    kin[1] = *reinterpret_cast<const u32x4*>(p.k + src + 8);
    vin[0] = *reinterpret_cast<const u32x4*>(p.v + src);
    vin[1] = *reinterpret_cast<const u32x4*>(p.v + src + 8);
    u32x4 kout = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t w = kin[e >> 3][(e >> 1) & 3];
      const uint32_t code = e4m3_code(bf16_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu)), p.k_inv);
      kout[e >> 2] |= code << (8 * (e & 3));
    }
    __builtin_nontemporal_store(kout, reinterpret_cast<u32x4*>(kdst));
    if constexpr (QUEST) {
      uint32_t key[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) key[e] = e4m3_bf16_bits((kout[e >> 2] >> (8 * (e & 3))) & 0xFFu);
      update_summary<16>(p, blk, h, dg, off == 0, key);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t w = vin[e >> 3][(e >> 1) & 3];
      const uint32_t code = e4m3_code(bf16_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu)), p.v_inv);
      __builtin_nontemporal_store((uint8_t)code, vtile + v_elem<4>(dg * 16 + e, r));
    }
  }
}

// One thread per (token, kv head, group of X elements).
template <bool FP8, bool QUEST>
__global__ __launch_bounds__(256) void cache_write_kernel(const CacheWriteParams p) {
  constexpr int X = FP8 ? 16 : 8;
  const int groups = p.head_dim / X;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)p.num_kv_heads * groups;
  if (gid >= (int64_t)p.num_tokens * per_token) return;
  const int j = (int)(gid / per_token);
  const int rem = (int)(gid - (int64_t)j * per_token);
  const int h = rem / groups;
  write_group<FP8, QUEST>(p, j, h, rem - h * groups);
}

// Bulk writes (a prefill's prompt rows): most tokens come in runs that fill
// whole 16-token sub-blocks, and those are written as whole tiles, K and V
// alike, with 16-byte stores on consecutive bytes: every cache line is
// written whole by one workgroup, instead of the per-token kernel's 2-byte
// V stores spread over the whole V tile.
//
// A workgroup (4 wavefronts) takes the token indices [16g, 16g + 16).  Token
// j is in a run when the 16 tokens a .. a + 15, a = j - slot[j] % 16, go to
// the slots b .. b + 15 of one sub-block (b = slot[a], b % 16 == 0; block
// sizes are multiples of 16).  The workgroup whose range holds a writes the
// run; the tokens of its range in no run are written one group at a time as
// the per-token kernel writes them.  Runs are decided from the slots alone,
// so every workgroup comes to the same answer for a token, and each token is
// written exactly once.
//
// A run is written head by head, one head per wavefront: its 16 K rows and
// 16 V rows (16 x D bf16 each) are staged in the wavefront's part of LDS
// with coalesced 16-byte loads (rows padded by 16 bytes so that the V
// gather below spreads over all banks), then each lane assembles whole
// 16-byte pieces of the two tiles: a K piece is 16 bytes of one token's row
// (8 bf16, or 16 dims as e4m3 codes); a V piece is 4 tokens x R dims
// (R = 2 bf16, or 4 e4m3 codes), [(d / 16) % R][t % 4] of the V layout.
template <int D, bool FP8>
__global__ __launch_bounds__(256) void cache_write_tiles_kernel(const CacheWriteParams p) {
  constexpr int X = FP8 ? 16 : 8;       // elements per 16-byte K piece
  constexpr int R = FP8 ? 4 : 2;        // dims per V piece row
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int RC = D / 8 + 1;         // staged row pitch in 16-byte chunks (padded)
  constexpr int TILE = kSub * D * EB;   // bytes of one K (or V) tile
  __shared__ u32x4 stage[4][2][kSub * RC];
  const int T = p.num_tokens;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j0 = blockIdx.x * kSub;

  // Lanes 0..15: token j0 + lane, its slot, whether it lies in a run and
  // whether it starts one.  Every wavefront computes the same.
  bool covered = false, anchor = false;
  if (lane < kSub && j0 + lane < T) {
    const int j = j0 + lane;
    const int64_t s = p.slots[j];
    if (s >= 0 && s < p.num_slots) {
      const int a = j - (int)(s & (kSub - 1));
      const int64_t base = s - (s & (kSub - 1));
      if (a >= 0 && a + kSub <= T) {
        bool ok = true;
        for (int k = 0; k < kSub; ++k) ok &= p.slots[a + k] == base + k;
        covered = ok;
        anchor = ok && a == j;
      }
    }
  }
  const uint64_t anchors = __ballot(anchor);
  const uint64_t singles = __ballot(lane < kSub && j0 + lane < T && !covered);

  if (anchors) {
    const int a = j0 + __builtin_ctzll(anchors);
    const int64_t b = p.slots[a];
    const int64_t blk = b / p.block_size;
    const int sub = (int)(b - blk * p.block_size) / kSub;
    const int subs = p.block_size / kSub;
    u32x4* ks = stage[wave][0];
    u32x4* vs = stage[wave][1];
    for (int h0 = 0; h0 < p.num_kv_heads; h0 += 4) {
      const int h = h0 + wave;
      const bool act = h < p.num_kv_heads;
      if (act) {
        // Stage: chunk c = (token t, 16-byte chunk cc of the head's row).
#pragma unroll
        for (int c = lane; c < kSub * (D / 8); c += 64) {
          const int t = c / (D / 8), cc = c % (D / 8);
          const int64_t src = ((int64_t)(a + t) * p.num_kv_heads + h) * D + cc * 8;
          ks[t * RC + cc] = *reinterpret_cast<const u32x4*>(p.k + src);
          vs[t * RC + cc] = *reinterpret_cast<const u32x4*>(p.v + src);
        }
      }
      __syncthreads();
      if (act) {
        const int64_t tile = ((blk * p.num_kv_heads + h) * subs + sub) * (int64_t)TILE;
        u32x4* kd = reinterpret_cast<u32x4*>(p.k_cache + tile);
        u32x4* vd = reinterpret_cast<u32x4*>(p.v_cache + tile);
        // K piece i = (d / X) * 16 + t: 16 bytes of token t's row.
#pragma unroll
        for (int i = lane; i < TILE / 16; i += 64) {
          const int t = i % kSub, pc = i / kSub;
          u32x4 out;
          if constexpr (FP8) {
            const u32x4 in[2] = {ks[t * RC + 2 * pc], ks[t * RC + 2 * pc + 1]};
            out = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const uint32_t w = in[e >> 3][(e >> 1) & 3];
              out[e >> 2] |= e4m3_code(bf16_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu)), p.k_inv) << (8 * (e & 3));
            }
          } else {
            out = ks[t * RC + pc];
          }
          __builtin_nontemporal_store(out, kd + i);
        }
        // V piece i = ((d / 16R) * 16 + d % 16) * 4 + t / 4, element
        // e = ((d / 16) % R) * 4 + t % 4.
        const uint16_t* v16 = reinterpret_cast<const uint16_t*>(vs);
#pragma unroll
        for (int i = lane; i < TILE / 16; i += 64) {
          const int t4 = i % 4, d16 = (i / 4) % 16, dq = i / 64;
          uint32_t x[4 * R];
#pragma unroll
          for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
              x[rr * 4 + tt] = v16[(t4 * 4 + tt) * RC * 8 + dq * 16 * R + rr * 16 + d16];
          u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 4 * R; ++e) {
            if constexpr (FP8)
              out[e >> 2] |= e4m3_code(bf16_to_f32(x[e]), p.v_inv) << (8 * (e & 3));
            else
              out[e >> 1] |= x[e] << (16 * (e & 1));
          }
          __builtin_nontemporal_store(out, vd + i);
        }
      }
      __syncthreads();
    }
  }

  // Tokens of the range in no run, one (token, head, group) per thread.
  if (singles) {
    const int groups = D / X;
    const int per_token = p.num_kv_heads * groups;
    const int n = __popcll(singles) * per_token;
    for (int i = threadIdx.x; i < n; i += 256) {
      const int k = i / per_token, rem = i - k * per_token;
      uint64_t m = singles;
      for (int q = 0; q < k; ++q) m &= m - 1;
      const int h = rem / groups;
      write_group<FP8, false>(p, j0 + __builtin_ctzll(m), h, rem - h * groups);
    }
  }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, bool fp8, hipStream_t stream) {
  const int X = fp8 ? 16 : 8;
  const int64_t threads = (int64_t)p.num_tokens * p.num_kv_heads * (p.head_dim / X);
  if (threads == 0) return hipSuccess;
  // Calls of a few hundred tokens (a decode step's new tokens, one per
  // sequence) rarely fill a sub-block and need all the parallelism they can
  // get: one thread per 16-byte group.  Larger calls look for whole
  // sub-blocks.  Both kernels store the same bytes.
  if (!p.summaries && p.num_tokens >= kTileWriteMinTokens) {
    const dim3 grid((unsigned)((p.num_tokens + kSub - 1) / kSub));
    if (p.head_dim == 128) {
      if (fp8)
        hipLaunchKernelGGL((cache_write_tiles_kernel<128, true>), grid, dim3(256), 0, stream, p);
      else
        hipLaunchKernelGGL((cache_write_tiles_kernel<128, false>), grid, dim3(256), 0, stream, p);
    } else {
      if (fp8)
        hipLaunchKernelGGL((cache_write_tiles_kernel<64, true>), grid, dim3(256), 0, stream, p);
      else
        hipLaunchKernelGGL((cache_write_tiles_kernel<64, false>), grid, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (p.summaries) {
    if (fp8)
      hipLaunchKernelGGL((cache_write_kernel<true, true>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((cache_write_kernel<false, true>), grid, dim3(256), 0, stream, p);
  } else {
    if (fp8)
      hipLaunchKernelGGL((cache_write_kernel<true, false>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((cache_write_kernel<false, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pa
