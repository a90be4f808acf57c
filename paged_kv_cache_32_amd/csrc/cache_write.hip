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
// The write is a few hundred bytes per token: it is latency bound, so the
// kernel is one thread per 16-byte K chunk of a (token, kv head) row, with
// the matching V elements, and no attempt at more.  A token's K row and V
// column write many cache lines in part (16-byte K pieces 256 bytes apart, V
// elements spread over the whole V tile); the stores carry the non-temporal
// hint so that those lines are not kept in L2 as partly written lines when
// the decode then streams the cache through it.
#include "pa_internal.h"

namespace pa {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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

// One thread per (token, kv head, group of X elements), X = 16 bytes of
// cache: 8 bf16 values or 16 fp8 codes.  QUEST: also the summary words of
// those X dimensions.
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
  const int dg = rem - h * groups;

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

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, bool fp8, hipStream_t stream) {
  const int X = fp8 ? 16 : 8;
  const int64_t threads = (int64_t)p.num_tokens * p.num_kv_heads * (p.head_dim / X);
  if (threads == 0) return hipSuccess;
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
