// Paged-attention decode for gfx950: one query token per sequence, grouped
// query heads, K/V gathered through the block table, split across
// wavefronts with a log-sum-exp merge.
//
// What is computed ("Taming the token torrent", "The Block Table Logic" and
// "Custom PagedAttention Kernels"; "KV Cache Engineering for LLM Serving",
// section 1): for sequence s and query head i reading KV head
// h = i / G, out = softmax(scale * q K^T) V over the sequence's tokens, with
// token t read from block block_tables[s][t / block_size].
//
// How (the pages' kernel sketch gives one thread block per (sequence, head)
// and stages each block in shared memory; this is a different design for
// CDNA4):
//  * Work unit = a wavefront.  The G query heads that share a KV head are a
//    16-wide MFMA operand, so each K/V byte is read once per (sequence,
//    KV head) and feeds all G heads.  The wavefront keeps its whole softmax
//    state (running max, running sum, 16 x head_dim accumulator) in
//    registers; no LDS and no barriers.
//  * A 16-token sub-block of one KV head is one contiguous tile in the cache
//    layout, ordered so that every load is a fully coalesced 16-byte
//    (K) or 8-/4-byte (V) per-lane load that lands directly in the MFMA
//    operand registers: K tile [d/X][16][X] gives lane (t, k-group) the 8
//    consecutive d of token t; V tile [d][16] gives lane (d, t-group) 4
//    consecutive tokens of dim d.
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (rows = tokens, cols = query
//    heads, fp32 accumulate; bf16 products are exact).  O^T = V^T P^T with
//    v_mfma_f32_16x16x16_bf16; P is split into a bf16 high part and a bf16
//    remainder so the probabilities keep ~16 significant bits.  fp8 codes
//    are widened to bf16 exactly on load.
//  * Online softmax in base 2 (scale * log2 e folded into the logit scale),
//    one max/rescale per stage of NSUB sub-blocks; cross-lane reductions
//    use 2 xor shuffles.
//  * Load balance: all (sequence, KV head) units are laid end to end as a
//    list of 16-token chunks, and wavefront w takes chunks
//    [w*C, (w+1)*C).  A unit that a wavefront covers completely is written
//    to `out` directly; a piece of a unit is written as a partial softmax
//    state (acc[G][D], m[G], l[G], padded to G * (D + 4) floats so records
//    stay 16-byte aligned).  Each piece is counted in with an agent-scope
//    atomic once its (coherent, write-through) stores have completed; the
//    wavefront that stores the last piece of a unit merges them (out = sum e^(m_p - M) acc_p / sum e^(m_p - M)
//    l_p) and re-arms the counter to zero, so one kernel launch does the
//    whole decode.  Every wavefront scans seq_lens itself, so there is no
//    planning kernel and no host synchronisation.
#include "pa_internal.h"

// Sub-blocks loaded per online-softmax step, and the fewest wavefronts per
// SIMD the register allocation must leave room for.
#ifndef PA_DECODE_STAGE
#define PA_DECODE_STAGE 4
#endif
#ifndef PA_DECODE_MIN_WAVES
#define PA_DECODE_MIN_WAVES 1
#endif
// 1: K/V tiles are read with the non-temporal hint (read once, no reuse).
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif

namespace pa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

__device__ __forceinline__ int wave_reduce_sum(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// Chunks (16-token pieces) of a sequence; -1 marks an invalid length.
__device__ __forceinline__ int chunks_of(int L, int max_len) {
  if (L < 0 || L > max_len) return -1;
  return (L + kSub - 1) / kSub;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ i16x4 as_i16x4(u32x2 v) { return __builtin_bit_cast(i16x4, v); }

// Two e4m3fn codes (bytes 0-1, or 2-3 when HI) -> two bf16, exactly.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Pack four probabilities into two bf16 operands: hi = p truncated to bf16,
// lo = (p - hi) truncated to bf16, so hi + lo = p to about 2^-16 relative.
__device__ __forceinline__ void split_p(const float p[4], i16x4& hi, i16x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = __float_as_uint(p[i]);
    h[i] = b;
    l[i] = __float_as_uint(p[i] - __uint_as_float(b & 0xFFFF0000u));
  }
  u32x2 H, Lo;
  H[0] = (h[0] >> 16) | (h[1] & 0xFFFF0000u);
  H[1] = (h[2] >> 16) | (h[3] & 0xFFFF0000u);
  Lo[0] = (l[0] >> 16) | (l[1] & 0xFFFF0000u);
  Lo[1] = (l[2] >> 16) | (l[3] & 0xFFFF0000u);
  hi = as_i16x4(H);
  lo = as_i16x4(Lo);
}

template <typename V>
__device__ __forceinline__ V load_kv(const V* p) {
#if PA_DECODE_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

template <int D, bool FP8>
struct Tile {
  static constexpr int EB = FP8 ? 1 : 2;           // bytes per cache element
  static constexpr int TILE_BYTES = kSub * D * EB;  // one (block, head, sub-block) tile
  static constexpr int KLD = FP8 ? D / 64 : D / 32; // 16-byte K loads per lane per tile
  static constexpr int QK = D / 32;                 // 16x16x32 MFMAs per tile (QK^T)
  static constexpr int DC = D / 16;                 // 16x16x16 MFMAs per tile (PV), per P half
  using VReg = typename std::conditional<FP8, uint32_t, u32x2>::type;
};

// State of one wavefront working on one (sequence, KV head) unit.
template <int D>
struct Softmax {
  float m;        // running max of base-2 logits of query head (lane & 15)
  float l;        // this lane's share of the running sum
  f32x4 acc[D / 16];
};

template <int D, bool FP8, int NSUB>
__device__ __forceinline__ void run_stage(const DecodeParams& p, int cnt, const uint8_t* const* kt,
                                          const uint8_t* const* vt, const bf16x8* qop,
                                          int first_tok, int L, Softmax<D>& st, int lane) {
  using T = Tile<D, FP8>;
  const int qd = lane >> 4, col = lane & 15;

  u32x4 kr[NSUB][T::KLD];
  typename T::VReg vr[NSUB][T::DC];
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    if (k < cnt) {
#pragma unroll
      for (int c = 0; c < T::KLD; ++c)
        kr[k][c] = load_kv(reinterpret_cast<const u32x4*>(kt[k] + c * 1024 + lane * 16));
#pragma unroll
      for (int dc = 0; dc < T::DC; ++dc) {
        if constexpr (FP8)
          vr[k][dc] = load_kv(reinterpret_cast<const uint32_t*>(vt[k] + dc * 256 + col * 16 + qd * 4));
        else
          vr[k][dc] = load_kv(reinterpret_cast<const u32x2*>(vt[k] + dc * 512 + col * 32 + qd * 8));
      }
    }
  }

  // Logits, base 2: lane holds tokens 4*qd + i of each sub-block, head col.
  float z[NSUB][4];
  float mx = kNegInf;
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    if (k < cnt) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FP8) {
#pragma unroll
        for (int c = 0; c < T::KLD; ++c) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 w;
            w[0] = fp8x2_to_bf16x2<false>(kr[k][c][2 * half]);
            w[1] = fp8x2_to_bf16x2<true>(kr[k][c][2 * half]);
            w[2] = fp8x2_to_bf16x2<false>(kr[k][c][2 * half + 1]);
            w[3] = fp8x2_to_bf16x2<true>(kr[k][c][2 * half + 1]);
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w), qop[2 * c + half], s, 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < T::QK; ++c)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[k][c]), qop[c], s, 0, 0, 0);
      }
      const int tok0 = first_tok + k * kSub + qd * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = s[i] * p.qk_scale;
        z[k][i] = (tok0 + i < L) ? v : kNegInf;
        mx = __builtin_fmaxf(mx, z[k][i]);
      }
    }
  }
  mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float m_new = __builtin_fmaxf(st.m, mx);
  const float alpha = (st.m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(st.m - m_new);
  st.m = m_new;

  float psum = 0.f;
  float pz[NSUB][4];
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    if (k < cnt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pz[k][i] = __builtin_amdgcn_exp2f(z[k][i] - m_new);
        psum += pz[k][i];
      }
    }
  }
  st.l = st.l * alpha + psum;
#pragma unroll
  for (int dc = 0; dc < T::DC; ++dc) st.acc[dc] *= alpha;

#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    if (k < cnt) {
      i16x4 phi, plo;
      split_p(pz[k], phi, plo);
      // Tokens past the sequence end hold arbitrary bits (possibly NaN):
      // their probability is 0, but 0 * NaN is NaN, so zero their V.
      const int tok0 = first_tok + k * kSub + qd * 4;
      const bool tail = (first_tok + k * kSub + kSub > L);
#pragma unroll
      for (int dc = 0; dc < T::DC; ++dc) {
        u32x2 a;
        if constexpr (FP8) {
          a[0] = fp8x2_to_bf16x2<false>(vr[k][dc]);
          a[1] = fp8x2_to_bf16x2<true>(vr[k][dc]);
        } else {
          a = vr[k][dc];
        }
        if (tail) {
          const uint32_t m0 = (tok0 + 0 < L ? 0x0000FFFFu : 0u) | (tok0 + 1 < L ? 0xFFFF0000u : 0u);
          const uint32_t m1 = (tok0 + 2 < L ? 0x0000FFFFu : 0u) | (tok0 + 3 < L ? 0xFFFF0000u : 0u);
          a[0] &= m0;
          a[1] &= m1;
        }
        const i16x4 av = as_i16x4(a);
        st.acc[dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, phi, st.acc[dc], 0, 0, 0);
        st.acc[dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, plo, st.acc[dc], 0, 0, 0);
      }
    }
  }
}

// Partial records are shared between wavefronts that may sit on different
// XCDs, whose L2 caches are not coherent with each other.  They are written
// and read with agent-scope atomic accesses, which the gfx950 memory system
// keeps coherent per instruction (write-through stores, L2-bypassing loads),
// so no cache-wide write-back or invalidate is needed: a writer waits for its
// stores to complete (s_waitcnt) before counting its piece in, and the merger
// only loads after it has read the counter.
__device__ __forceinline__ void store_shared(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_shared(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the partial softmax states of unit (s, h), pieces from wavefronts
// w0..w1, into out (run by the wavefront that stored the last piece):
// out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p, M = max_p m_p.
template <int D>
__device__ __forceinline__ void merge_unit(const DecodeParams& p, int s, int h, int64_t u0,
                                           int64_t w0, int64_t w1, int64_t C, int lane) {
  const int G = p.group;
  const int64_t rec_len = (int64_t)G * (D + 4);
  float* o = p.out + ((int64_t)s * p.num_q_heads + (int64_t)h * G) * D;
  const int vec = G * D / 4;
  for (int e = lane; e < vec; e += 64) {
    const int g = e / (D / 4), d4 = e - g * (D / 4);
    float M = kNegInf;
    for (int64_t w = w0; w <= w1; ++w) {
      const int64_t slot = (w == w0 && u0 != w0 * C) ? 2 * w + 1 : 2 * w;
      M = __builtin_fmaxf(M, load_shared(p.partials + slot * rec_len + (int64_t)G * D + g));
    }
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    for (int64_t w = w0; w <= w1; ++w) {
      const int64_t slot = (w == w0 && u0 != w0 * C) ? 2 * w + 1 : 2 * w;
      const float* rec = p.partials + slot * rec_len;
      const float m = load_shared(rec + (int64_t)G * D + g);
      const float f = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m - M);
      const float* a = rec + (int64_t)g * D + d4 * 4;
      num += f * f32x4{load_shared(a), load_shared(a + 1), load_shared(a + 2), load_shared(a + 3)};
      den += f * load_shared(rec + (int64_t)G * D + G + g);
    }
    reinterpret_cast<f32x4*>(o)[e] = num * (p.out_scale / den);
  }
}

template <int D, bool FP8, int NSUB>
__global__ __launch_bounds__(kDecodeThreads, PA_DECODE_MIN_WAVES) void decode_kernel(const DecodeParams p) {
  using T = Tile<D, FP8>;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  if (wave >= p.num_waves) return;
  const int S = p.num_seqs, Hkv = p.num_kv_heads, G = p.group;
  const int max_len = p.max_blocks * p.block_size;
  const int subs = p.block_size / kSub;

  // Pass 1: total chunks.  Wavefront 0 also writes the rows no other
  // wavefront will touch: zeros for empty sequences, NaN for invalid ones.
  int64_t total = 0;
  for (int base = 0; base < S; base += 64) {
    const int si = base + lane;
    int n = 0;
    if (si < S) n = chunks_of(p.seq_lens[si], max_len);
    if (wave == 0) {
      uint64_t todo = __ballot(si < S && n <= 0);
      while (todo) {
        const int l0 = __builtin_ctzll(todo);
        todo &= todo - 1;
        const float v = (readlane(n, l0) < 0) ? __builtin_nanf("") : 0.f;
        float* o = p.out + (int64_t)(base + l0) * p.num_q_heads * D;
        for (int e = lane; e < p.num_q_heads * D / 4; e += 64)
          reinterpret_cast<f32x4*>(o)[e] = f32x4{v, v, v, v};
      }
    }
    n = n < 0 ? 0 : n;
    total += wave_reduce_sum(n);
  }
  const int64_t W = total * Hkv;
  int64_t C = p.chunk_fixed;
  if (C <= 0) {
    C = (W + p.num_waves - 1) / p.num_waves;
    if (C < p.chunk_min) C = p.chunk_min;
  }
  const int64_t a = (int64_t)wave * C;
  if (a >= W) return;
  const int64_t b = (a + C < W) ? a + C : W;

  // Pass 2: the sequence holding chunk a.
  int s = 0;
  int64_t before = 0;  // chunks of the sequences before s (per KV head)
  {
    int64_t carry = 0;
    for (int base = 0; base < S; base += 64) {
      const int si = base + lane;
      int n = 0;
      if (si < S) n = chunks_of(p.seq_lens[si], max_len);
      n = n < 0 ? 0 : n;
      const int incl = wave_incl_scan(n, lane);
      const int64_t lo = (int64_t)Hkv * (carry + incl - n), hi = (int64_t)Hkv * (carry + incl);
      const uint64_t hit = __ballot(n > 0 && lo <= a && a < hi);
      if (hit) {
        const int l0 = __builtin_ctzll(hit);
        s = base + l0;
        before = carry + readlane(incl - n, l0);
        break;
      }
      carry += readlane(incl, 63);
    }
  }

  const int qd = lane >> 4, col = lane & 15;
  int64_t x = a;
  while (x < b && s < S) {
    const int L = p.seq_lens[s];
    const int n = chunks_of(L, max_len);
    if (n <= 0) { ++s; continue; }
    const int64_t u0s = (int64_t)Hkv * before;
    const int64_t off = x - u0s;
    const int h = (int)(off / n);
    const int j0 = (int)(off - (int64_t)h * n);
    const int64_t u0 = u0s + (int64_t)h * n;
    const int64_t uend = u0 + n;
    const int64_t seg_end = (b < uend) ? b : uend;
    const int j1 = j0 + (int)(seg_end - x);

    // Query operand: lane (col = head in group, qd = k-group) holds 8 dims.
    bf16x8 qop[T::QK];
    {
      const uint16_t* qrow = p.q + ((int64_t)s * p.num_q_heads + (int64_t)h * G + col) * D;
#pragma unroll
      for (int c = 0; c < T::QK; ++c) {
        // bf16 K tiles put dims 32c + 8qd .. +7 in MFMA c; fp8 K tiles put
        // dims 64(c/2) + 16qd + 8(c%2) .. +7 there.
        const int d0 = FP8 ? 64 * (c >> 1) + 16 * qd + 8 * (c & 1) : 32 * c + 8 * qd;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (col < G) w = *reinterpret_cast<const u32x4*>(qrow + d0);
        qop[c] = as_bf16x8(w);
      }
    }

    Softmax<D> st;
    st.m = kNegInf;
    st.l = 0.f;
#pragma unroll
    for (int dc = 0; dc < T::DC; ++dc) st.acc[dc] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks;
    const int nblk = (L + p.block_size - 1) / p.block_size;
    int win_base = INT32_MIN / 2;
    int win = -1;
    bool bad = false;
    const int64_t head_tiles = (int64_t)h * subs;
    for (int j = j0; j < j1;) {
      const int cnt = (j1 - j < NSUB) ? (j1 - j) : NSUB;
      const uint8_t* kt[NSUB];
      const uint8_t* vt[NSUB];
#pragma unroll
      for (int k = 0; k < NSUB; ++k) {
        kt[k] = p.k_cache;
        vt[k] = p.v_cache;
        if (k < cnt) {
          const int jj = j + k;
          const int bi = jj / subs;
          const int sub = jj - bi * subs;
          if (bi - win_base >= 64 || bi < win_base) {
            win_base = bi;
            const int e = win_base + lane;
            win = (e < nblk) ? bt[e] : -1;
          }
          const int blk = readlane(win, bi - win_base);
          if ((unsigned)blk < (unsigned)p.num_blocks) {
            const int64_t tile = ((int64_t)blk * Hkv * subs + head_tiles + sub) * T::TILE_BYTES;
            kt[k] = p.k_cache + tile;
            vt[k] = p.v_cache + tile;
          } else {
            bad = true;
          }
        }
      }
      run_stage<D, FP8, NSUB>(p, cnt, kt, vt, qop, j * kSub, L, st, lane);
      j += cnt;
    }

    float ltot = st.l + __shfl_xor(st.l, 16, 64);
    ltot += __shfl_xor(ltot, 32, 64);
    if (bad) ltot = __builtin_nanf("");
    const bool complete = (j0 == 0 && j1 == n);
    if (complete) {
      if (col < G) {
        const float inv = p.out_scale / ltot;
        float* o = p.out + ((int64_t)s * p.num_q_heads + (int64_t)h * G + col) * D + qd * 4;
#pragma unroll
        for (int dc = 0; dc < T::DC; ++dc) *reinterpret_cast<f32x4*>(o + dc * 16) = st.acc[dc] * inv;
      }
    } else {
      // Store this piece, then count it in; the wavefront that stores the
      // unit's last piece merges all of them and re-arms the counter.
      const int64_t slot = (x == a) ? 2 * (int64_t)wave : 2 * (int64_t)wave + 1;
      float* rec = p.partials + slot * (int64_t)G * (D + 4);
      if (col < G) {
        float* o = rec + (int64_t)col * D + qd * 4;
#pragma unroll
        for (int dc = 0; dc < T::DC; ++dc)
#pragma unroll
          for (int i = 0; i < 4; ++i) store_shared(o + dc * 16 + i, st.acc[dc][i]);
        if (qd == 0) {
          store_shared(rec + (int64_t)G * D + col, st.m);
          store_shared(rec + (int64_t)G * D + G + col, ltot);
        }
      }
      const int64_t w0 = u0 / C, w1 = (uend - 1) / C;
      int32_t* counter = p.counters + (int64_t)s * Hkv + h;
      __builtin_amdgcn_s_waitcnt(0);  // this wavefront's record stores have completed
      int prior = 0;
      if (lane == 0) prior = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      prior = readlane(prior, 0);
      if (prior == (int)(w1 - w0)) {
        merge_unit<D>(p, s, h, u0, w0, w1, C, lane);
        if (lane == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }

    x = seg_end;
    if (x == uend && h == Hkv - 1) {
      before += n;
      ++s;
    }
  }
}

constexpr int kStage = PA_DECODE_STAGE;

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

template <int D, bool FP8>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream) {
  const unsigned groups = (unsigned)((p.num_waves + kWavesPerGroup - 1) / kWavesPerGroup);
  hipLaunchKernelGGL((decode_kernel<D, FP8, kStage>), dim3(groups), dim3(kDecodeThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool FP8>
int resident_waves_typed() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<D, FP8, kStage>, kDecodeThreads, 0) !=
      hipSuccess)
    return 0;
  return cus * per_cu * kWavesPerGroup;
}

}  // namespace

hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t stream) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<uint32_t*>(ptr), words);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, bool fp8, hipStream_t stream) {
  if (p.head_dim == 128) return fp8 ? launch_typed<128, true>(p, stream) : launch_typed<128, false>(p, stream);
  if (p.head_dim == 64) return fp8 ? launch_typed<64, true>(p, stream) : launch_typed<64, false>(p, stream);
  return hipErrorInvalidValue;
}

int decode_resident_waves(int head_dim, bool fp8) {
  if (head_dim == 128) return fp8 ? resident_waves_typed<128, true>() : resident_waves_typed<128, false>();
  if (head_dim == 64) return fp8 ? resident_waves_typed<64, true>() : resident_waves_typed<64, false>();
  return 0;
}

}  // namespace pa
