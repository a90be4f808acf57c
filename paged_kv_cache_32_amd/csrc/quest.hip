// Query-aware page selection (Quest) over the paged cache ("KV Cache
// Engineering for LLM Serving", section 7, Query-aware sparse reads).
//
// A page is one cache block.  Each (block, KV head) keeps, per key
// dimension, the minimum and the maximum of the keys stored in it; a new
// query scores every page of its sequence by the largest q.k any key inside
// that min/max box could reach, sum_d max(q_d min_d, q_d max_d), and only the
// best `budget` pages are then read by the decode.
//
// Summary words: one uint32 per (block, head, dim), bits 0-15 the minimum
// and bits 16-31 the maximum, both as bf16 (every stored key is exactly a
// bf16 value: a bf16 key, or an e4m3 code's value without the per-tensor
// scale), laid out [block][dim / 4][head][4] (summary_word in
// pa_internal.h).  An empty summary is min = +inf, max = -inf.  The cache
// write can keep them itself (pa_quest_cache_write, cache_write.hip).
//
// Kernels:
//   summary_fill_kernel    every word empty (a plain fill, graph-safe).
//   summary_reset_kernel   words of blocks written at offset 0 in this call
//                          become empty (a block's first token starts it).
//   summary_merge_kernel   each written token's stored key widens its
//                          block's words (compare-and-swap per word).
//   summary_build_kernel   words of listed blocks recomputed from their
//                          first `count` tokens (after a copy or swap-in).
//   page_score_kernel      score of every page of every (sequence, KV head),
//                          as an order-preserving uint32 key (a workgroup
//                          per run of a sequence's pages, all KV heads).
//   page_select_kernel     per (sequence, KV head): the `budget` best pages
//                          (equal scores: lower page first) by a radix select
//                          on the keys, written in page order as a compacted
//                          block table, with the token count it covers.
// The decode over the compacted tables is the paged decode kernel itself,
// run with one "sequence" per (sequence, KV head).
#include "pa_internal.h"

namespace pa {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kEmptyWord = kEmptySummaryWord;

__device__ __forceinline__ float bf16f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// bf16 bits of an e4m3fn code's value (no scale): exact.  NaN codes give a
// bf16 NaN.
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 8;
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  if (e == 15u && m == 7u) return sign | 0x7FC0u;
  if (e == 0u) return sign | (__float_as_uint((float)m * 0x1p-9f) >> 16);
  return sign | ((e + 120u) << 7) | (m << 4);
}

// Widens one summary word by a key value (bf16 bits); NaN keys are ignored.
// Ranges only grow inside one launch, so a word that already covers the
// value needs no write.
__device__ __forceinline__ void widen(uint32_t* w, uint32_t vb) {
  const float v = bf16f(vb);
  if (v != v) return;
  uint32_t old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    const uint32_t lo = old & 0xFFFFu, hi = old >> 16;
    const bool lower = v < bf16f(lo), higher = v > bf16f(hi);
    if (!lower && !higher) return;
    const uint32_t nw = ((higher ? vb : hi) << 16) | (lower ? vb : lo);
    if (__hip_atomic_compare_exchange_strong(w, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return;
  }
}

__global__ __launch_bounds__(256) void summary_fill_kernel(u32x4* words, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) words[i] = u32x4{kEmptyWord, kEmptyWord, kEmptyWord, kEmptyWord};
}

// One thread per (token, head, 4 words).
__global__ __launch_bounds__(256) void summary_reset_kernel(const SummaryParams p) {
  const int q4 = p.head_dim / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_token = (int64_t)p.num_kv_heads * q4;
  if (gid >= (int64_t)p.num_tokens * per_token) return;
  const int j = (int)(gid / per_token);
  const int rem = (int)(gid - (int64_t)j * per_token);
  const int h = rem / q4, i = rem - h * q4;
  const int64_t slot = p.slots[j];
  if (slot < 0 || slot >= (int64_t)p.num_blocks * p.block_size || slot % p.block_size != 0) return;
  const int64_t blk = slot / p.block_size;
  u32x4* w = reinterpret_cast<u32x4*>(p.words + summary_word(blk, h, 4 * i, p.num_kv_heads, p.head_dim));
  *w = u32x4{kEmptyWord, kEmptyWord, kEmptyWord, kEmptyWord};
}

// bf16 bits of element e of a 16-byte K chunk.
template <bool FP8>
__device__ __forceinline__ uint32_t chunk_elem(const u32x4& c, int e) {
  if constexpr (FP8) return e4m3_to_bf16((c[e >> 2] >> (8 * (e & 3))) & 0xFFu);
  return (c[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
}

// Byte offset of the 16-byte K chunk (block, head, token, chunk dg): the
// cache layout [blk][h][t / 16][d / X][t % 16][X elements].
__device__ __forceinline__ int64_t k_chunk(const SummaryParams& p, int64_t blk, int h, int t, int dg,
                                           int eb) {
  const int subs = p.block_size / kSub;
  const int64_t tile = ((blk * p.num_kv_heads + h) * subs + t / kSub) * (int64_t)(kSub * p.head_dim) * eb;
  return tile + ((int64_t)dg * kSub + t % kSub) * 16;
}

// One thread per (token, head, 16-byte chunk of the key).
template <bool FP8>
__global__ __launch_bounds__(256) void summary_merge_kernel(const SummaryParams p) {
  constexpr int X = FP8 ? 16 : 8;
  const int groups = p.head_dim / X;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_token = (int64_t)p.num_kv_heads * groups;
  if (gid >= (int64_t)p.num_tokens * per_token) return;
  const int j = (int)(gid / per_token);
  const int rem = (int)(gid - (int64_t)j * per_token);
  const int h = rem / groups, dg = rem - h * groups;
  const int64_t slot = p.slots[j];
  if (slot < 0 || slot >= (int64_t)p.num_blocks * p.block_size) return;
  const int64_t blk = slot / p.block_size;
  const int t = (int)(slot - blk * p.block_size);
  const u32x4 c = *reinterpret_cast<const u32x4*>(p.k_cache + k_chunk(p, blk, h, t, dg, FP8 ? 1 : 2));
#pragma unroll
  for (int e = 0; e < X; ++e)
    widen(p.words + summary_word(blk, h, dg * X + e, p.num_kv_heads, p.head_dim), chunk_elem<FP8>(c, e));
}

// One thread per (listed block, head, 16-byte chunk): min and max over the
// block's first count tokens, then one store per word.
template <bool FP8>
__global__ __launch_bounds__(256) void summary_build_kernel(const SummaryParams p) {
  constexpr int X = FP8 ? 16 : 8;
  const int groups = p.head_dim / X;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_item = (int64_t)p.num_kv_heads * groups;
  if (gid >= (int64_t)p.num_tokens * per_item) return;
  const int i = (int)(gid / per_item);
  const int rem = (int)(gid - (int64_t)i * per_item);
  const int h = rem / groups, dg = rem - h * groups;
  const int blk = p.blocks[i];
  if ((unsigned)blk >= (unsigned)p.num_blocks) return;
  int count = p.counts[i];
  count = count < 0 ? 0 : (count > p.block_size ? p.block_size : count);
  uint32_t lo[X], hi[X];
#pragma unroll
  for (int e = 0; e < X; ++e) {
    lo[e] = 0x7F80u;
    hi[e] = 0xFF80u;
  }
  for (int t = 0; t < count; ++t) {
    const u32x4 c = *reinterpret_cast<const u32x4*>(p.k_cache + k_chunk(p, blk, h, t, dg, FP8 ? 1 : 2));
#pragma unroll
    for (int e = 0; e < X; ++e) {
      const uint32_t vb = chunk_elem<FP8>(c, e);
      const float v = bf16f(vb);
      if (v < bf16f(lo[e])) lo[e] = vb;
      if (v > bf16f(hi[e])) hi[e] = vb;
    }
  }
#pragma unroll
  for (int v = 0; v < X / 4; ++v)
    *reinterpret_cast<u32x4*>(p.words + summary_word(blk, h, dg * X + 4 * v, p.num_kv_heads, p.head_dim)) =
        u32x4{(hi[4 * v] << 16) | lo[4 * v], (hi[4 * v + 1] << 16) | lo[4 * v + 1],
              (hi[4 * v + 2] << 16) | lo[4 * v + 2], (hi[4 * v + 3] << 16) | lo[4 * v + 3]};
}

// Order-preserving uint32 of a score: a larger key is a larger score; -0 is
// +0, and NaN takes the lowest key.
__device__ __forceinline__ uint32_t score_key(float x) {
  if (x != x) return 0u;
  const uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Pages of sequence s, or -1 for a length outside [0, max_blocks * bs].
__device__ __forceinline__ int pages_of(const SelectParams& p, int s) {
  const int L = p.seq_lens[s];
  if (L < 0 || (int64_t)L > (int64_t)p.max_blocks * p.block_size) return -1;
  return (L + p.block_size - 1) / p.block_size;
}

__device__ __forceinline__ int wave_incl_sum(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// Score workgroups: kScoreWaves wavefronts that share the staged queries of
// one sequence.  A lane scores kScorePages pages of one KV head; lanes
// (slot, head) with the heads fastest, so the lanes of a page read one run
// of the block's summary words (all heads' quads of 4 dimensions, 128 bytes
// at 8 heads) per load instruction.  kScoreAhead dimension quads of every
// page are in flight while the previous ones are summed.  Every LDS read of
// a q+ / q- quad serves the lane's kScorePages pages (at 8 heads, a read of
// 8 distinct quads takes the LDS as long as a full 1 KiB read).  Two pages
// per lane keep a workgroup's item at 64 pages: four halved those reads but
// left a batch of 64 sequences, or of 4 sequences of 8,192 pages, with
// fewer items than the two workgroups per CU can hold.
#ifndef PA_SCORE_PAGES
#define PA_SCORE_PAGES 2
#endif
#ifndef PA_SCORE_LDS_FLOATS
#define PA_SCORE_LDS_FLOATS 16384
#endif
#ifndef PA_SCORE_AHEAD
#define PA_SCORE_AHEAD 2
#endif
#ifndef PA_SCORE_GROUPS_PER_CU
#define PA_SCORE_GROUPS_PER_CU 2
#endif
constexpr int kScoreWaves = 4;
constexpr int kScoreThreads = 64 * kScoreWaves;
constexpr int kScorePages = PA_SCORE_PAGES;
constexpr int kScoreAhead = PA_SCORE_AHEAD;
constexpr int kScoreLdsFloats = PA_SCORE_LDS_FLOATS;   // q+ and q- of the staged heads
constexpr int kScoreGroupsPerCu = PA_SCORE_GROUPS_PER_CU;

// Work item: the item_pages pages c * item_pages .. of sequence s (a
// sequence of n pages has ceil(n / item_pages) items, numbered in sequence
// order); workgroups stride over the items.  Per item and slice of
// slice_heads KV heads, the workgroup stages q+ = max(q, 0) and q- =
// min(q, 0) of the slice's query heads in LDS as float32, the group padded
// to GP heads with zeros: q+ in the first half of the array and q- in the
// second, each as [KV head][query head][quad of 4 dimensions], the quad
// index XORed with the KV head, so that the 8 heads' lanes of one read land
// in 8 different 16-byte slots of every 128 bytes (no bank conflicts) while
// a lane's reads of one step differ by constant offsets.  Each lane then sums, for every query head of its group,
// over the dimensions in order, in float32: for a page's min <= max and a
// query value q, max(q * min, q * max) is q * max when q >= 0 and q * min
// otherwise, so the term is added as two fused multiply-adds, acc =
// fma(q+, max, acc) then acc = fma(q-, min, acc), one of which adds a zero.
// A product of two bf16 values is exact in float32 whenever its magnitude
// is at least 2^-134, so this rounds exactly as a rounded product and a
// rounded sum would (a zero's sign aside, which never changes a sum's
// value).  The page's score is the largest sum of the group.
template <int D, int GP>
__global__ __launch_bounds__(kScoreThreads) void page_score_kernel(const SelectParams p) {
  __shared__ __attribute__((aligned(16))) float qs[kScoreLdsFloats];
  constexpr int Q4 = D / 4;                       // dimension quads
  // Quads per batch: at most kScoreAhead, fewer for 16 query heads (more
  // registers per quad), and at most a quarter of a page so that the loop
  // below runs at least twice (a loop of one pass becomes straight-line code
  // whose hoisted addresses the compiler then spills).
  constexpr int PP = kScorePages;
  constexpr int PF0 = GP >= 16 ? kScoreAhead / 2 : kScoreAhead;
  constexpr int PF = PF0 < Q4 / 4 ? PF0 : Q4 / 4;
  static_assert(Q4 % (2 * PF) == 0 && Q4 / (2 * PF) >= 2, "the batch loop runs at least twice");
  const int Hkv = p.num_kv_heads, G = p.group, Hs = p.slice_heads, PI = p.item_pages;
  const int S = p.num_seqs;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int slots = 64 / Hs;                      // page slots per wavefront
  const int hh = lane % Hs, slot = lane / Hs;
  const int gq = GP * Q4;                         // quads per staged KV head (in each of q+ and q-)
  for (int it = blockIdx.x;; it += gridDim.x) {
    // The item's sequence (every wavefront finds the same one).
    int s = -1, c = 0, np = 0;
    {
      int carry = 0;
      for (int base = 0; base < S; base += 64) {
        const int si = base + lane;
        int npl = 0, n = 0;
        if (si < S) {
          npl = pages_of(p, si);
          n = npl > 0 ? (npl + PI - 1) / PI : 0;
        }
        const int incl = wave_incl_sum(n, lane);
        const uint64_t hit = __ballot(n > 0 && carry + incl - n <= it && it < carry + incl);
        if (hit) {
          const int l0 = __builtin_ctzll(hit);
          s = base + l0;
          c = it - (carry + __builtin_amdgcn_readlane(incl - n, l0));
          np = __builtin_amdgcn_readlane(npl, l0);
          break;
        }
        carry += __builtin_amdgcn_readlane(incl, 63);
      }
    }
    if (s < 0) break;                              // past the last item: the same for the whole workgroup
    const int pg0 = c * PI + wv * slots * PP;      // this wavefront's first page
    int blk[PP];
    bool live[PP], ok[PP];
#pragma unroll
    for (int k = 0; k < PP; ++k) {
      const int pg = pg0 + k * slots + slot;
      live[k] = slot < slots && pg < np;
      blk[k] = live[k] ? p.block_tables[(int64_t)s * p.max_blocks + pg] : 0;
      ok[k] = (unsigned)blk[k] < (unsigned)p.num_blocks;
      if (!ok[k]) blk[k] = 0;                      // read block 0 in its place; the page scores lowest
    }
    for (int h0 = 0; h0 < Hkv; h0 += Hs) {
      const int hn = Hkv - h0 < Hs ? Hkv - h0 : Hs;
      const int h = h0 + (hh < hn ? hh : 0);
      const u32x4* row[PP];
#pragma unroll
      for (int k = 0; k < PP; ++k)
        row[k] = reinterpret_cast<const u32x4*>(p.words + summary_word(blk[k], h, 0, Hkv, D));
      // Quad j of a page's head h sits Hkv quads after quad j - 1.  The
      // loads are non-temporal: a call reads each summary line once, and
      // from HBM (a step's other reads evict the summaries between calls)
      // they measured faster than cached loads.
      auto load = [&](u32x4 (&v)[PF][PP], int j0) {
#pragma unroll
        for (int jj = 0; jj < PF; ++jj) {
          const int j = j0 + jj < Q4 ? j0 + jj : Q4 - 1;   // past the end: a repeat, never summed
#pragma unroll
          for (int k = 0; k < PP; ++k) v[jj][k] = __builtin_nontemporal_load(&row[k][(int64_t)j * Hkv]);
        }
      };
      float acc[PP][GP];
#pragma unroll
      for (int k = 0; k < PP; ++k)
#pragma unroll
        for (int g = 0; g < GP; ++g) acc[k][g] = 0.f;
      const float* qh = qs + (hh < hn ? hh : 0) * gq * 4;
      const int sw = (hh < hn ? hh : 0) & 7;
      auto sum = [&](const u32x4 (&v)[PF][PP], int j0) {
#pragma unroll
        for (int jj = 0; jj < PF; ++jj) {
          const int j = j0 + jj;
          const int jx = (j ^ sw) * 4;
          float mn[PP][4], mx[PP][4];
#pragma unroll
          for (int k = 0; k < PP; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              mn[k][e] = __uint_as_float(v[jj][k][e] << 16);
              mx[k][e] = __uint_as_float(v[jj][k][e] & 0xFFFF0000u);
            }
#pragma unroll
          for (int g = 0; g < GP; ++g) {
            const float* qq = qh + g * Q4 * 4 + jx;
            const float4 qp = *reinterpret_cast<const float4*>(qq);
            const float4 qn = *reinterpret_cast<const float4*>(qq + kScoreLdsFloats / 2);
            const float qpa[4] = {qp.x, qp.y, qp.z, qp.w}, qna[4] = {qn.x, qn.y, qn.z, qn.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int k = 0; k < PP; ++k) {
                acc[k][g] = __builtin_fmaf(qpa[e], mx[k][e], acc[k][g]);
                acc[k][g] = __builtin_fmaf(qna[e], mn[k][e], acc[k][g]);
              }
          }
        }
      };
      // The first batch of this slice's summary loads is issued before the
      // queries are staged, so their latencies overlap.  The scheduling
      // barriers keep each batch of loads where it is issued (without them
      // the compiler sinks every load to just before its use, and each quad
      // then waits a whole memory latency).
      u32x4 va[PF][PP], vb[PF][PP];
      load(va, 0);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();                             // the previous slice's reads of qs are done
      // Staging: each thread takes 8 dimensions (16 bytes of q) at a time,
      // kStageLoads of them with all loads issued before the first is used.
      const uint16_t* qseq = p.q + (int64_t)s * p.num_q_heads * D;
      constexpr int kStageLoads = 4;
      const int octs = hn * gq / 2;                 // 8-dimension runs of the slice's query heads
      for (int i0 = tid; i0 < octs; i0 += kScoreThreads * kStageLoads) {
        u32x4 raw[kStageLoads];
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
          const int i = i0 + u * kScoreThreads;
          const int hs = i / (gq / 2), rem = i - hs * (gq / 2), g = rem / (Q4 / 2), jp = rem - g * (Q4 / 2);
          // Runs past the slice or the group read the sequence's first run
          // instead (always inside q) and are zeroed below.
          const bool in = i < octs && g < G;
          raw[u] = *reinterpret_cast<const u32x4*>(qseq + (in ? ((h0 + hs) * G + g) * D + 8 * jp : 0));
          if (!in) raw[u] = u32x4{0u, 0u, 0u, 0u};
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
          const int i = i0 + u * kScoreThreads;
          if (i < octs) {
            const int hs = i / (gq / 2), rem = i - hs * (gq / 2), g = rem / (Q4 / 2), jp = rem - g * (Q4 / 2);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int j = 2 * jp + half;
              const uint32_t w0 = raw[u][2 * half], w1 = raw[u][2 * half + 1];
              const uint32_t b[4] = {w0 & 0xFFFFu, w0 >> 16, w1 & 0xFFFFu, w1 >> 16};
              float4 qp, qn;
              float* pp = &qp.x;
              float* pn = &qn.x;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float qf = __uint_as_float(b[e] << 16);
                pp[e] = (b[e] & 0x8000u) ? 0.f : qf;
                pn[e] = (b[e] & 0x8000u) ? qf : 0.f;
              }
              float* dst = qs + ((hs * GP + g) * Q4 + (j ^ (hs & 7))) * 4;
              *reinterpret_cast<float4*>(dst) = qp;
              *reinterpret_cast<float4*>(dst + kScoreLdsFloats / 2) = qn;
            }
          }
        }
      }
      __syncthreads();
#pragma unroll 1
      for (int j0 = 0; j0 < Q4; j0 += 2 * PF) {
        load(vb, j0 + PF);
        __builtin_amdgcn_sched_barrier(0);
        sum(va, j0);
        __builtin_amdgcn_sched_barrier(0);
        load(va, j0 + 2 * PF);
        __builtin_amdgcn_sched_barrier(0);
        sum(vb, j0 + PF);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int k = 0; k < PP; ++k) {
        if (live[k] && hh < hn) {
          uint32_t key = 0u;  // a block outside the pool scores lowest
          if (ok[k]) {
            float best = -__builtin_inff();
#pragma unroll
            for (int g = 0; g < GP; ++g)
              if (g < G) best = __builtin_fmaxf(best, acc[k][g]);
            key = score_key(best);
          }
          p.keys[((int64_t)s * Hkv + h) * p.max_blocks + pg0 + k * slots + slot] = key;
        }
      }
    }
  }
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum of v over the 256 threads (red: 4 ints of LDS; two barriers).
template <int NW>
__device__ __forceinline__ int block_sum(int v, int* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += red[i];
  __syncthreads();
  return t;
}

// Exclusive prefix sums in thread order of two small counts a, e in [0, 64)
// and the block's total of a, with one exchange through `scratch` (2 * NW
// words, not read again by the caller before a barrier).  Within a
// wavefront each bit of a count is counted over the lower lanes with a
// ballot and mbcnt (set bits below the lane) and over the wavefront with a
// scalar popcount, so the wavefront needs no cross-lane data movement.
template <int NW>
__device__ __forceinline__ void block_excl_sum2_small(int a, int e, int* scratch, int& a_before, int& e_before,
                                                      int& a_total) {
  int ba = 0, be = 0, ta = 0, te = 0;
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const uint64_t ma = __ballot((a >> b) & 1), me = __ballot((e >> b) & 1);
    ba += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(ma >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ma, 0u)) << b;
    be += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, 0u)) << b;
    ta += __popcll(ma) << b;
    te += __popcll(me) << b;
  }
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    scratch[wv] = ta;
    scratch[NW + wv] = te;
  }
  __syncthreads();
  int pa = 0, pe = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int x = scratch[i], y = scratch[NW + i];
    pa += i < wv ? x : 0;
    pe += i < wv ? y : 0;
    tot += x;
  }
  a_before = pa + ba;
  e_before = pe + be;
  a_total = tot;
}

// Exclusive prefix sum of v over the 256 threads in thread order.
__device__ __forceinline__ int block_excl_sum(int v, int* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int incl = wave_incl_sum(v, lane);
  if (lane == 63) red[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < wv; ++i) before += red[i];
  __syncthreads();
  return before + incl - v;
}

// Keys of up to kSelectLds pages are kept in LDS, one pad word per 32 so
// that threads walking contiguous ranges hit different banks; longer
// sequences read them from global memory (where the score kernel just
// wrote them).
constexpr int kSelectLds = 12288;
constexpr int kSelectRegs = 32;   // keys per thread held in registers (pages <= 8192)
__device__ __forceinline__ int lds_index(int i) { return i + (i >> 5); }

// Workgroup per unit (s, h): the budget best pages by key, equal keys to the
// lower page; written in page order to sel_tables[unit][0..budget), with
// sel_lens[unit] = tokens they hold.
//
// The threshold T = the budget-th largest key is found from the top: 8 bits
// per round with an LDS histogram for units held in registers with at most
// 16 keys per thread, else bit by bit (32 counting rounds: T keeps a bit
// when at least `budget` keys are >= T with it; for units held in registers
// a wavefront counts with one ballot per key slot and scalar popcounts).
// Then each thread takes a contiguous range of pages: the
// pages above T, and the first (budget - count above T) pages equal to T,
// go to their place in page order through two prefix sums.
//
// The workgroup has NT threads: 256, or 1,024 when the tables are wider than
// 2,048 pages (a long unit's keys then spread over four times the threads).
// Units of up to NT * REGS pages keep everything in registers: the
// keys (strided, for counting), and the keys and block ids of the thread's
// own contiguous range (for the compaction).  All of those loads are issued
// before the counting rounds, so their latency is paid once.  Longer units
// read keys from LDS or global memory in each round.
template <int NT, int REGS>
__device__ __forceinline__ void select_small(const SelectParams& p, int unit, int s, int np,
                                             const uint32_t* gk, uint32_t* lk, int* red, uint32_t* hist) {
  const int tid = threadIdx.x;
  const int B = p.budget;
  int32_t* out = p.sel_tables + (int64_t)unit * B;
  const int32_t* row = p.block_tables + (int64_t)s * p.max_blocks;
  const int m = (np + NT - 1) / NT;                     // <= REGS
  const int i0 = tid * m < np ? tid * m : np;
  const int cnt = np - i0 < m ? np - i0 : m;
  uint32_t kr[REGS];
  int32_t ids[REGS];
#pragma unroll
  for (int k = 0; k < REGS; ++k) kr[k] = tid + NT * k < np ? gk[tid + NT * k] : 0u;
#pragma unroll
  for (int k = 0; k < REGS; ++k) ids[k] = k < cnt ? row[i0 + k] : -1;
#pragma unroll
  for (int k = 0; k < REGS; ++k)
    if (tid + NT * k < np) lk[lds_index(tid + NT * k)] = kr[k];
  // T = the budget-th largest key.  Units of at most 16 key slots per
  // thread find it 8 bits per round from the top of the keys' range: with
  // x = key - (the unit's smallest key), which orders the keys as they are,
  // the keys whose x agrees with T's above the round's digit are counted per
  // digit value (LDS histogram); T takes the largest digit with at least
  // `want` of them at or above it, and `want` drops by those strictly above.
  // Taking the digits from the range rather than from bit 31 matters: one
  // unit's keys share their top bits (the sign and exponent range of its
  // scores), which would crowd the first round into a few bins, and the LDS
  // atomics on one bin serialize.  Fuller units find T bit by bit: T keeps
  // a bit when at least `budget` keys are >= T with it, counted with one
  // ballot per key slot and scalar popcounts.
  const int slots = (np + NT - 1) / NT;     // key slots that hold any page
  uint32_t T = 0u;
  if (slots <= 16) {
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int k = 0; k < REGS; ++k) {
      if (k < slots && tid + NT * k < np) {
        kmn = kr[k] < kmn ? kr[k] : kmn;
        kmx = kr[k] > kmx ? kr[k] : kmx;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint32_t a = (uint32_t)__shfl_xor((int)kmn, o, 64), b = (uint32_t)__shfl_xor((int)kmx, o, 64);
      kmn = a < kmn ? a : kmn;
      kmx = b > kmx ? b : kmx;
    }
    // Two histogram buffers alternate between rounds: while wavefront 0
    // scans one, the other threads clear the next, so a round needs two
    // barriers.  The block's minimum and maximum pass through the second.
    if (tid < 256) hist[tid] = 0u;
    if ((tid & 63) == 0) {
      hist[256 + (tid >> 6)] = kmn;
      hist[256 + 64 + (tid >> 6)] = kmx;
    }
    __syncthreads();                            // also publishes the LDS keys
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      kmn = hist[256 + i] < kmn ? hist[256 + i] : kmn;
      kmx = hist[256 + 64 + i] > kmx ? hist[256 + 64 + i] : kmx;
    }
    const int nbits = kmx > kmn ? 32 - __builtin_clz(kmx - kmn) : 0;
    uint32_t X = 0u;                            // T - kmn
    int want = B;
    int r = 0;
    for (int hi = nbits; hi > 0; hi -= 8, ++r) {
      const int lo = hi > 8 ? hi - 8 : 0;
      const uint32_t dmask = (1u << (hi - lo)) - 1u;
      uint32_t* cur = hist + 256 * (r & 1);
      uint32_t* nxt = hist + 256 * ((r + 1) & 1);
      int* rr = red + 2 * (r & 1);
#pragma unroll
      for (int k = 0; k < REGS; ++k) {
        if (k < slots && tid + NT * k < np) {
          const uint32_t x = kr[k] - kmn;
          const bool match = hi == nbits || ((x ^ X) >> hi) == 0u;
          if (match) atomicAdd(&cur[(x >> lo) & dmask], 1u);
        }
      }
      __syncthreads();
      for (int i = tid - 64; i >= 0 && i < 256; i += NT - 64) nxt[i] = 0u;
      if (tid < 64) {
        // Lane l holds digits 4l .. 4l + 3; suffix sums from the top digit.
        uint32_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = cur[4 * tid + i];
        const int own = (int)(h[0] + h[1] + h[2] + h[3]);
        int suf = own;                          // sum over lanes >= tid
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int u = __shfl_down(suf, o, 64);
          if (tid + o < 64) suf += u;
        }
        // S(d) for this lane's digits, top first; the largest d with S(d) >= want.
        int above = suf - own;                  // keys in digits above 4 tid + 3
        int dbest = -1, above_best = 0;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          const int Sd = above + (int)h[i];
          if (dbest < 0 && Sd >= want) {
            dbest = 4 * tid + i;
            above_best = above;
          }
          above = Sd;
        }
        const uint64_t hit = __ballot(dbest >= 0);
        const int l = 63 - __builtin_clzll(hit);  // the highest lane with a qualifying digit
        if (tid == l) {
          rr[0] = dbest;
          rr[1] = want - above_best;
        }
      }
      // Every thread has read the previous round's results (before this
      // round's first barrier), so those slots are free again next round.
      __syncthreads();
      X |= (uint32_t)rr[0] << lo;
      want = rr[1];
    }
    T = X + kmn;
  } else {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);   // >= 1: the padding keys 0 never count
      int c = 0;
#pragma unroll
      for (int k = 0; k < REGS; ++k) c += __popcll(__ballot(kr[k] >= cand));
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
      __syncthreads();                        // also publishes the LDS keys
      int total = 0;
#pragma unroll
      for (int i = 0; i < NT / 64; ++i) total += red[i];
      __syncthreads();
      if (total >= B) T = cand;
    }
  }
  uint32_t mine[REGS];
  int above = 0, equal = 0;
#pragma unroll
  for (int k = 0; k < REGS; ++k) {
    mine[k] = k < cnt ? lk[lds_index(i0 + k)] : 0u;
    above += (k < cnt && mine[k] > T) ? 1 : 0;
    equal += (k < cnt && mine[k] == T) ? 1 : 0;
  }
  // One scan gives the keys above T and equal to it in the ranges before
  // this thread's, and the block's keys above T.  The keys equal to T are
  // taken in page order until `need` of them are, so the thread's first
  // output position is (above before) + min(equal before, need).  The
  // scratch words are the histogram's, which nothing reads any more (the
  // last round, or the bit rounds, ended with a barrier).
  int above_before, eq_before, above_total;
  block_excl_sum2_small<NT / 64>(above, equal, reinterpret_cast<int*>(hist), above_before, eq_before,
                                 above_total);
  const int need = B - above_total;
  int pos = above_before + (eq_before < need ? eq_before : need);
  int er = eq_before;
  const int last_valid = p.seq_lens[s] - (np - 1) * p.block_size;
#pragma unroll
  for (int k = 0; k < REGS; ++k) {
    if (k < cnt) {
      const bool eq = mine[k] == T;
      const bool take = mine[k] > T || (eq && er < need);
      er += eq ? 1 : 0;
      if (take && pos < B) {
        out[pos] = ids[k];
        ++pos;
      }
      if (i0 + k == np - 1) p.sel_lens[unit] = take ? (B - 1) * p.block_size + last_valid : B * p.block_size;
    }
  }
}

template <int NT, bool LDS>
__device__ __forceinline__ void select_unit(const SelectParams& p, int unit, int s, int np, const uint32_t* gk,
                                            uint32_t* lk, int* red) {
  const int tid = threadIdx.x;
  const int B = p.budget;
  int32_t* out = p.sel_tables + (int64_t)unit * B;
  const int32_t* row = p.block_tables + (int64_t)s * p.max_blocks;
  auto key = [&](int i) -> uint32_t {
    if constexpr (LDS) return lk[lds_index(i)];
    return gk[i];
  };
  uint32_t T = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
    for (int i = tid; i < np; i += NT) c += key(i) >= cand ? 1 : 0;
    if (block_sum<NT / 64>(c, red) >= B) T = cand;
  }
  // Contiguous ranges: thread t owns pages [t * m, min(np, (t + 1) * m)).
  const int m = (np + NT - 1) / NT;
  const int i0 = tid * m < np ? tid * m : np, i1 = (tid + 1) * m < np ? (tid + 1) * m : np;
  int above = 0, equal = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t k = key(i);
    above += k > T ? 1 : 0;
    equal += k == T ? 1 : 0;
  }
  const int need = B - block_sum<NT / 64>(above, red);
  const int eq_rank0 = block_excl_sum(equal, red);
  int taken = 0;
  {
    int er = eq_rank0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = key(i);
      const bool eq = k == T;
      taken += (k > T || (eq && er < need)) ? 1 : 0;
      er += eq ? 1 : 0;
    }
  }
  int pos = block_excl_sum(taken, red);
  int er = eq_rank0;
  const int last_valid = p.seq_lens[s] - (np - 1) * p.block_size;
  for (int i = i0; i < i1; ++i) {
    const uint32_t k = key(i);
    const bool eq = k == T;
    const bool take = k > T || (eq && er < need);
    er += eq ? 1 : 0;
    if (take && pos < B) {
      out[pos] = row[i];
      ++pos;
    }
    if (i == np - 1) p.sel_lens[unit] = take ? (B - 1) * p.block_size + last_valid : B * p.block_size;
  }
}

// Units whose pages all fit the budget copy their table row; invalid
// lengths give sel_lens = -1.
template <int NT>
__global__ __launch_bounds__(NT) void page_select_kernel(const SelectParams p) {
  constexpr int REGS = NT == 1024 ? 12 : kSelectRegs;   // NT * REGS <= kSelectLds keys held in LDS
  __shared__ uint32_t lk[kSelectLds + kSelectLds / 32];
  __shared__ int red[NT / 64];
  __shared__ uint32_t hist[512];
  const int unit = blockIdx.x;
  const int s = unit / p.num_kv_heads;
  const int tid = threadIdx.x;
  const int B = p.budget;
  const int np = pages_of(p, s);
  if (np < 0 || np <= B) {
    int32_t* out = p.sel_tables + (int64_t)unit * B;
    const int32_t* row = p.block_tables + (int64_t)s * p.max_blocks;
    for (int i = tid; i < B; i += NT) out[i] = (np >= 0 && i < np) ? row[i] : -1;
    if (tid == 0) p.sel_lens[unit] = np < 0 ? -1 : p.seq_lens[s];
    return;
  }
  const uint32_t* gk = p.keys + (int64_t)unit * p.max_blocks;
  if (np <= NT * REGS) {
    select_small<NT, REGS>(p, unit, s, np, gk, lk, red, hist);
  } else if (np <= kSelectLds) {
    // Eight independent loads in flight per thread before their stores.
    for (int i0 = tid; i0 < np; i0 += 8 * NT) {
      uint32_t v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = i0 + NT * k < np ? gk[i0 + NT * k] : 0u;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (i0 + NT * k < np) lk[lds_index(i0 + NT * k)] = v[k];
    }
    __syncthreads();
    select_unit<NT, true>(p, unit, s, np, gk, lk, red);
  } else {
    select_unit<NT, false>(p, unit, s, np, gk, lk, red);
  }
}

}  // namespace

hipError_t launch_summary_fill(uint32_t* words, int64_t n_words, hipStream_t stream) {
  const int64_t n4 = n_words / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(summary_fill_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<u32x4*>(words), n4);
  return hipGetLastError();
}

hipError_t launch_summary_update(const SummaryParams& p, bool fp8, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  const int64_t reset_threads = (int64_t)p.num_tokens * p.num_kv_heads * (p.head_dim / 4);
  hipLaunchKernelGGL(summary_reset_kernel, dim3((unsigned)((reset_threads + 255) / 256)), dim3(256), 0,
                     stream, p);
  const int64_t merge_threads = (int64_t)p.num_tokens * p.num_kv_heads * (p.head_dim / (fp8 ? 16 : 8));
  const dim3 grid((unsigned)((merge_threads + 255) / 256));
  if (fp8)
    hipLaunchKernelGGL(summary_merge_kernel<true>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(summary_merge_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_summary_build(const SummaryParams& p, bool fp8, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  const int64_t threads = (int64_t)p.num_tokens * p.num_kv_heads * (p.head_dim / (fp8 ? 16 : 8));
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (fp8)
    hipLaunchKernelGGL(summary_build_kernel<true>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(summary_build_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D>
void launch_score(const SelectParams& p, int gp, dim3 grid, hipStream_t stream) {
  switch (gp) {
    case 1: hipLaunchKernelGGL((page_score_kernel<D, 1>), grid, dim3(kScoreThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((page_score_kernel<D, 2>), grid, dim3(kScoreThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((page_score_kernel<D, 4>), grid, dim3(kScoreThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((page_score_kernel<D, 8>), grid, dim3(kScoreThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL((page_score_kernel<D, 16>), grid, dim3(kScoreThreads), 0, stream, p); break;
  }
}

hipError_t launch_page_select(const SelectParams& p_in, hipStream_t stream) {
  const int64_t units = (int64_t)p_in.num_seqs * p_in.num_kv_heads;
  if (units == 0) return hipSuccess;
  SelectParams p = p_in;
  // Query heads per group padded to a power of two; KV heads whose queries
  // fit the 64 KiB of LDS at once (and a page's heads fit a wavefront).
  int gp = 1;
  while (gp < p.group) gp *= 2;
  int hs = kScoreLdsFloats / (2 * gp * p.head_dim);   // q+ and q- of hs KV heads
  if (hs > 64) hs = 64;
  if (hs > p.num_kv_heads) hs = p.num_kv_heads;
  p.slice_heads = hs;
  p.item_pages = kScoreWaves * (64 / hs) * kScorePages;
  // Two workgroups per CU (their LDS fills 128 KiB of the 160); no more than
  // the items there can be.
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  const int64_t most = (int64_t)p.num_seqs * ((p.max_blocks + p.item_pages - 1) / p.item_pages);
  int64_t groups = kScoreGroupsPerCu * (int64_t)cus;
  if (groups > most) groups = most;
  if (groups > 0) {
    const dim3 grid((unsigned)groups);
    if (p.head_dim == 128)
      launch_score<128>(p, gp, grid, stream);
    else
      launch_score<64>(p, gp, grid, stream);
  }
  // Wide tables: a 1,024-thread workgroup per unit (fewer keys per thread).
  if (p.max_blocks > 2048)
    hipLaunchKernelGGL(page_select_kernel<1024>, dim3((unsigned)units), dim3(1024), 0, stream, p);
  else
    hipLaunchKernelGGL(page_select_kernel<256>, dim3((unsigned)units), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
