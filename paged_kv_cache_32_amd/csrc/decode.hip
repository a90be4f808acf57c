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
//    per-lane load (1 KiB per instruction) that lands directly in the MFMA
//    operand registers: K tile [d/X][16][X] gives lane (t, k-group) the 8
//    consecutive d of token t; V tile [d/16R][d%16][t/4][(d/16)%R][t%4]
//    gives lane (d%16, t-group) 4 consecutive tokens of R dims 16 apart,
//    the V^T operand of R MFMAs.
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


// Values the whole wavefront agrees on, marked so for the compiler (so that
// control flow and the addresses of scalar loads stay in scalar registers).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Scalar (SMEM) loads of uniform indices: block ids and sequence lengths are
// read through the constant address space so they come back on the scalar
// counter, independent of the K/V loads in flight.
typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;
__device__ __forceinline__ int sload(const int32_t* base, int64_t i) {
  return ((const_i32_ptr)base)[i];
}

// Wait until at most N vector-memory operations of this wavefront are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int D, bool FP8>
struct Tile {
  static constexpr int EB = FP8 ? 1 : 2;           // bytes per cache element
  static constexpr int TILE_BYTES = kSub * D * EB;  // one (block, head, sub-block) tile
  static constexpr int KLD = FP8 ? D / 64 : D / 32; // 16-byte K loads per lane per tile
  static constexpr int QK = D / 32;                 // 16x16x32 MFMAs per tile (QK^T)
  static constexpr int DC = D / 16;                 // 16x16x16 MFMAs per tile (PV), per P half
  static constexpr int R = FP8 ? 4 : 2;             // PV MFMAs fed by one 16-byte V load
  static constexpr int VLD = DC / R;                // 16-byte V loads per lane per tile
};

// Registers one pipeline stage loads into: NSUB K and V tiles and the query
// operand of the stage's unit (used only when the stage starts a piece).
template <int D, bool FP8, int NSUB>
struct StageBuf {
  using T = Tile<D, FP8>;
  static constexpr int kLoads = NSUB * (T::KLD + T::VLD) + T::QK;  // per issue, always
  u32x4 k[NSUB][T::KLD];
  u32x4 v[NSUB][T::VLD];
  u32x4 q[T::QK];
};

// Softmax state of the unit piece a wavefront is working on.
template <int D>
struct Softmax {
  float m;        // running max of base-2 logits of query head (lane & 15)
  float l;        // this lane's share of the running sum
  f32x4 acc[D / 16];
};

// One stage of a wavefront's work, uniform across the wavefront: up to NSUB
// consecutive 16-token chunks of unit (s, h).
struct Stage {
  int s, h, j, cnt, L, n;
  int j_first;     // chunk (within the unit) where this wavefront's piece starts
  int64_t u0;      // linear index of the unit's first chunk
  bool valid;      // false past the end of the wavefront's range
  bool first;      // first stage of the piece: load Q, reset the softmax state
  bool last;       // last stage of the piece: write it out or store the partial
  bool piece_at_a; // the piece starts at the wavefront's first chunk
  bool bad;        // a block id of this stage is outside the pool
};

// Where a wavefront stands: chunk x of the linear list, chunk j of unit
// (s, h); the sub-range being walked ends at `end`.
struct Pos {
  int64_t x, end;
  int64_t before;  // chunks (per KV head) of the sequences before s
  int s, n, L, h, j;
};

// Uniform cursor over the wavefront's range [a, b), walked as up to three
// sub-ranges: the piece holding chunk a, the piece holding chunk b - 1, and
// the whole units between them.  The two boundary pieces (the ones another
// wavefront shares) go first, so that split units are merged early rather
// than at the end of the kernel.
struct Cursor {
  Pos cur;
  Pos queue[2];
  int nq;
  int64_t a;
  int j_first;
  int64_t piece_x;
  bool new_piece;
};

// A partial piece on its way to being counted in: stored (its stores must
// complete first), then counted (the counter's old value is in flight).
struct Pending {
  int state;       // 0 empty, 1 stored, 2 counted
  int s, h;
  int64_t u0, w0, w1;
  int prior;       // lane 0: counter value before this piece was counted
};

// Pieces of wavefront w are stored in slot 2w (the piece that starts at the
// wavefront's first chunk) or 2w + 1 (the piece that ends at its last).
__device__ __forceinline__ int64_t piece_slot(int64_t w, int64_t w0, int64_t u0, int64_t C) {
  return (w == w0 && u0 != w0 * C) ? 2 * w + 1 : 2 * w;
}

// Partial records are shared between wavefronts that may sit on different
// XCDs, whose L2 caches are not coherent with each other.  They are written
// and read with buffer accesses carrying the device-coherence cache bit
// (write-through stores, loads that miss the L2), so no cache-wide
// write-back or invalidate is needed: a writer counts its piece in only after
// its stores have completed (s_waitcnt), and the merger only loads after it
// has read the counter.  A record holds acc as [D/4][G][4] floats (16-byte
// pieces, lane-contiguous per store) and then {m, l, 0, 0} per query head.
constexpr int kDeviceCoherent = 16;           // sc1
constexpr int kBufferWord3 = 0x00020000;      // raw 32-bit buffer access
__device__ __forceinline__ __amdgpu_buffer_rsrc_t record_rsrc(const float* rec, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(rec), 0, bytes, kBufferWord3);
}
__device__ __forceinline__ void store_record(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, kDeviceCoherent);
}
__device__ __forceinline__ f32x4 load_record(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kDeviceCoherent));
}

// Merge the partial softmax states of unit (s, h), pieces from wavefronts
// w0..w1, into out (run by the wavefront that counted in the last piece):
// out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p, M = max_p m_p, taken
// one piece at a time with a running maximum.  Lane l handles the 4-float
// groups e = l + 64 i of the G x D output, kIt of them per pass; all loads of
// one piece for a pass are issued together.
template <int D>
__device__ __forceinline__ void merge_unit(const DecodeParams& p, const Pending& pd, int64_t C,
                                           int lane) {
  constexpr int kIt = 4;
  const int G = p.group;
  const int groups = G * D / 4;
  const int rec_bytes = G * (D + 4) * 4;
  f32x4* o = reinterpret_cast<f32x4*>(p.out + ((int64_t)pd.s * p.num_q_heads + (int64_t)pd.h * G) * D);
  for (int e0 = 0; e0 < groups; e0 += 64 * kIt) {
    float M[kIt], den[kIt];
    f32x4 num[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      M[it] = kNegInf;
      den[it] = 0.f;
      num[it] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int64_t w = pd.w0; w <= pd.w1; ++w) {
      const auto r = record_rsrc(p.partials + piece_slot(w, pd.w0, pd.u0, C) * (rec_bytes / 4), rec_bytes);
      f32x4 ml[kIt], acc[kIt];
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int e = e0 + lane + 64 * it;
        const int g = e / (D / 4), d4 = e - g * (D / 4);
        if (e < groups) {
          ml[it] = load_record(r, (G * D + g * 4) * 4);
          acc[it] = load_record(r, (d4 * G + g) * 16);
        }
      }
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        if (e0 + lane + 64 * it < groups) {
          const float m_new = __builtin_fmaxf(M[it], ml[it][0]);
          const float a = (M[it] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M[it] - m_new);
          const float f = (ml[it][0] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ml[it][0] - m_new);
          num[it] = num[it] * a + acc[it] * f;
          den[it] = den[it] * a + ml[it][1] * f;
          M[it] = m_new;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int e = e0 + lane + 64 * it;
      if (e < groups) o[e] = num[it] * (p.out_scale / den[it]);
    }
  }
}

// Count a stored piece in (its stores have completed).
__device__ __forceinline__ void count_piece(const DecodeParams& p, Pending& pd, int lane) {
  int32_t* counter = p.counters + (int64_t)pd.s * p.num_kv_heads + pd.h;
  pd.prior = 0;
  if (lane == 0) pd.prior = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  pd.state = 2;
}

// Read the counter's old value: the wavefront that counted in the unit's
// last piece merges all of them and re-arms the counter for the next call.
template <int D>
__device__ __forceinline__ void resolve_piece(const DecodeParams& p, Pending& pd, int64_t C, int lane) {
  const int prior = readlane(pd.prior, 0);
  if (prior == (int)(pd.w1 - pd.w0)) {
    merge_unit<D>(p, pd, C, lane);
    if (lane == 0)
      __hip_atomic_store(p.counters + (int64_t)pd.s * p.num_kv_heads + pd.h, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  pd.state = 0;
}

// The unit after the one p stands in (p.j reset to 0); seq_lens is read for
// the following sequences when p's was its sequence's last unit.
__device__ __forceinline__ void next_unit(Pos& c, const DecodeParams& p, int max_len) {
  c.j = 0;
  if (c.h + 1 < p.num_kv_heads) {
    ++c.h;
    return;
  }
  c.h = 0;
  c.before += c.n;
  // Only called while chunks remain, so a later sequence with chunks exists.
  for (;;) {
    ++c.s;
    c.L = sload(p.seq_lens, c.s);
    c.n = chunks_of(c.L, max_len);
    if (c.n > 0) break;
  }
}

// Next stage of the cursor's range; moves the cursor past it.
template <int NSUB>
__device__ __forceinline__ Stage next_stage(Cursor& cc, const DecodeParams& p, int max_len) {
  if (cc.cur.x >= cc.cur.end && cc.nq > 0) {
    cc.cur = cc.queue[0];
    cc.queue[0] = cc.queue[1];
    --cc.nq;
    cc.new_piece = true;
  }
  Pos& c = cc.cur;
  Stage st;
  st.valid = c.x < c.end;
  st.s = uni(c.s); st.h = uni(c.h); st.j = uni(c.j); st.L = uni(c.L); st.n = uni(c.n);
  st.u0 = uni64((int64_t)p.num_kv_heads * c.before + (int64_t)c.h * c.n);
  st.bad = false;
  st.first = cc.new_piece;
  if (cc.new_piece) {
    cc.j_first = c.j;
    cc.piece_x = c.x;
  }
  st.j_first = cc.j_first;
  st.piece_at_a = (cc.piece_x == cc.a);
  if (!st.valid) {
    st.cnt = 0;
    st.first = st.last = false;
    return st;
  }
  int64_t cnt = c.n - c.j;
  if (c.end - c.x < cnt) cnt = c.end - c.x;
  if (NSUB < cnt) cnt = NSUB;
  st.cnt = uni((int)cnt);
  c.x += cnt;
  c.j += (int)cnt;
  cc.new_piece = false;
  st.last = (c.j == c.n) || (c.x == c.end);
  if (c.j == c.n && c.x < c.end) {
    cc.new_piece = true;
    next_unit(c, p, max_len);
  }
  return st;
}

// Issue every load of a stage: exactly StageBuf::kLoads vector loads, always,
// so the wait counts the compiler derives do not depend on the branch taken.
// Chunk slots past the stage (or a stage past the range) read one fixed line.
template <int D, bool FP8, int NSUB>
__device__ __forceinline__ void issue_stage(const DecodeParams& p, Stage& st,
                                            StageBuf<D, FP8, NSUB>& buf, int lane) {
  using T = Tile<D, FP8>;
  const int qd = lane >> 4, col = lane & 15;
  const int G = p.group;
  const int subs = p.block_size / kSub;
  // Query operand: lane (col = head in group, qd = k-group) holds 8 dims.
  {
    const bool want = st.first && col < G;
    const uint16_t* qrow = p.q + ((int64_t)st.s * p.num_q_heads + (int64_t)st.h * G + col) * D;
#pragma unroll
    for (int c = 0; c < T::QK; ++c) {
      // bf16 K tiles put dims 32c + 8qd .. +7 in MFMA c; fp8 K tiles put
      // dims 64(c/2) + 16qd + 8(c%2) .. +7 there.
      const int d0 = FP8 ? 64 * (c >> 1) + 16 * qd + 8 * (c & 1) : 32 * c + 8 * qd;
      buf.q[c] = *reinterpret_cast<const u32x4*>(want ? qrow + d0 : p.q);
    }
  }
  const int32_t* bt = p.block_tables + (int64_t)st.s * p.max_blocks;
  const int64_t head_tiles = (int64_t)st.h * subs;
  // All block ids of the stage first (scalar loads, one wait), then the
  // tiles.  Chunk slots past the stage re-read the last valid id.
  int blk[NSUB];
  const int jlast = st.valid ? st.j + st.cnt - 1 : 0;
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    const int jj = (st.j + k < jlast) ? st.j + k : jlast;
    blk[k] = sload(bt, jj / subs);
  }
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    int64_t tile = 0;
    bool ok = false;
    if (k < st.cnt) {
      const int jj = st.j + k;
      const int bi = jj / subs;
      ok = (unsigned)blk[k] < (unsigned)p.num_blocks;
      if (ok)
        tile = ((int64_t)blk[k] * p.num_kv_heads * subs + head_tiles + (jj - bi * subs)) * T::TILE_BYTES;
      else
        st.bad = true;
    }
    const uint8_t* kt = p.k_cache + tile;
    const uint8_t* vt = p.v_cache + tile;
    const int kl = ok ? lane * 16 : 0;
    const int vl = ok ? (col * 4 + qd) * 16 : 0;
#pragma unroll
    for (int c = 0; c < T::KLD; ++c)
      buf.k[k][c] = load_kv(reinterpret_cast<const u32x4*>(kt + c * 1024 + kl));
    // V tile [d/16R][d%16][t/4][(d/16)%R][t%4]: lane (col, qd) reads the 16
    // bytes holding tokens 4qd..4qd+3 of dims 16(R e + r) + col.
#pragma unroll
    for (int e = 0; e < T::VLD; ++e)
      buf.v[k][e] = load_kv(reinterpret_cast<const u32x4*>(vt + e * 1024 + vl));
  }
}

// The math of one stage: logits, online-softmax update, P V accumulation.
template <int D, bool FP8, int NSUB>
__device__ __forceinline__ void compute_stage(const DecodeParams& p, const Stage& st,
                                              const StageBuf<D, FP8, NSUB>& buf,
                                              const bf16x8* qop, Softmax<D>& sm, int lane) {
  using T = Tile<D, FP8>;
  const int qd = lane >> 4;
  const int first_tok = st.j * kSub;
  const int L = st.L;

  // Logits, base 2: lane holds tokens 4*qd + i of each sub-block, head col.
  float z[NSUB][4];
  float mx = kNegInf;
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    if (k < st.cnt) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FP8) {
#pragma unroll
        for (int c = 0; c < T::KLD; ++c) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 w;
            w[0] = fp8x2_to_bf16x2<false>(buf.k[k][c][2 * half]);
            w[1] = fp8x2_to_bf16x2<true>(buf.k[k][c][2 * half]);
            w[2] = fp8x2_to_bf16x2<false>(buf.k[k][c][2 * half + 1]);
            w[3] = fp8x2_to_bf16x2<true>(buf.k[k][c][2 * half + 1]);
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w), qop[2 * c + half], s, 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < T::QK; ++c)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(buf.k[k][c]), qop[c], s, 0, 0, 0);
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
  const float m_new = __builtin_fmaxf(sm.m, mx);
  const float alpha = (sm.m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(sm.m - m_new);
  sm.m = m_new;

  float psum = 0.f;
  float pz[NSUB][4];
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    if (k < st.cnt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pz[k][i] = __builtin_amdgcn_exp2f(z[k][i] - m_new);
        psum += pz[k][i];
      }
    }
  }
  sm.l = sm.l * alpha + psum;
#pragma unroll
  for (int dc = 0; dc < T::DC; ++dc) sm.acc[dc] *= alpha;

#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    if (k < st.cnt) {
      i16x4 phi, plo;
      split_p(pz[k], phi, plo);
      // Tokens past the sequence end hold arbitrary bits (possibly NaN):
      // their probability is 0, but 0 * NaN is NaN, so zero their V.
      const int tok0 = first_tok + k * kSub + qd * 4;
      const bool tail = (first_tok + k * kSub + kSub > L);
      const uint32_t m0 = (tok0 + 0 < L ? 0x0000FFFFu : 0u) | (tok0 + 1 < L ? 0xFFFF0000u : 0u);
      const uint32_t m1 = (tok0 + 2 < L ? 0x0000FFFFu : 0u) | (tok0 + 3 < L ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int dc = 0; dc < T::DC; ++dc) {
        u32x2 a;
        if constexpr (FP8) {
          const uint32_t w = buf.v[k][dc / T::R][dc % T::R];
          a[0] = fp8x2_to_bf16x2<false>(w);
          a[1] = fp8x2_to_bf16x2<true>(w);
        } else {
          a[0] = buf.v[k][dc / T::R][2 * (dc % T::R)];
          a[1] = buf.v[k][dc / T::R][2 * (dc % T::R) + 1];
        }
        if (tail) {
          a[0] &= m0;
          a[1] &= m1;
        }
        const i16x4 av = as_i16x4(a);
        sm.acc[dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, phi, sm.acc[dc], 0, 0, 0);
        sm.acc[dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, plo, sm.acc[dc], 0, 0, 0);
      }
    }
  }
}

// Per-wavefront state carried across stages.
template <int D>
struct WaveState_ {
  Softmax<D> sm;
  bool bad;
  Pending pend[2];
};
template <int D, bool FP8>
struct WaveState : WaveState_<D> {
  bf16x8 q[Tile<D, FP8>::QK];
};

// Math of a stage plus, at a piece boundary, the piece's output.
template <int D, bool FP8, int NSUB>
__device__ __forceinline__ void finish_stage(const DecodeParams& p, const Stage& st,
                                             const StageBuf<D, FP8, NSUB>& buf,
                                             WaveState<D, FP8>& ws, int64_t wave, int64_t C,
                                             int lane) {
  using T = Tile<D, FP8>;
  if (!st.valid) return;
  const int qd = lane >> 4, col = lane & 15;
  const int G = p.group;
  if (st.first) {
#pragma unroll
    for (int c = 0; c < T::QK; ++c) ws.q[c] = as_bf16x8(col < G ? buf.q[c] : u32x4{0u, 0u, 0u, 0u});
    ws.sm.m = kNegInf;
    ws.sm.l = 0.f;
#pragma unroll
    for (int dc = 0; dc < T::DC; ++dc) ws.sm.acc[dc] = f32x4{0.f, 0.f, 0.f, 0.f};
    ws.bad = false;
  }
  ws.bad |= st.bad;
  compute_stage<D, FP8, NSUB>(p, st, buf, ws.q, ws.sm, lane);
  if (!st.last) return;

  float ltot = ws.sm.l + __shfl_xor(ws.sm.l, 16, 64);
  ltot += __shfl_xor(ltot, 32, 64);
  if (ws.bad) ltot = __builtin_nanf("");
  if (st.j_first == 0 && st.j + st.cnt == st.n) {
    // The whole unit is this wavefront's: write the output directly.
    if (col < G) {
      const float inv = p.out_scale / ltot;
      float* o = p.out + ((int64_t)st.s * p.num_q_heads + (int64_t)st.h * G + col) * D + qd * 4;
#pragma unroll
      for (int dc = 0; dc < T::DC; ++dc) *reinterpret_cast<f32x4*>(o + dc * 16) = ws.sm.acc[dc] * inv;
    }
    return;
  }
  const int64_t slot = st.piece_at_a ? 2 * wave : 2 * wave + 1;
  const int rec_bytes = G * (D + 4) * 4;
  const auto r = record_rsrc(p.partials + slot * (rec_bytes / 4), rec_bytes);
  if (col < G) {
#pragma unroll
    for (int dc = 0; dc < T::DC; ++dc) store_record(r, ((dc * 4 + qd) * G + col) * 16, ws.sm.acc[dc]);
    if (qd == 0) store_record(r, (G * D + col * 4) * 4, f32x4{ws.sm.m, ltot, 0.f, 0.f});
  }
  Pending& pd = (ws.pend[0].state == 0) ? ws.pend[0] : ws.pend[1];
  pd.state = 1;
  pd.s = st.s;
  pd.h = st.h;
  pd.u0 = st.u0;
  pd.w0 = st.u0 / C;
  pd.w1 = (st.u0 + st.n - 1) / C;
}

// Advance the pieces waiting to be counted in.  Called right after a
// stage's loads were issued: every piece stored before that issue has its
// stores complete once all but those loads are done, and every counter
// value read before it has arrived by then too.
template <int D, int LOADS>
__device__ __forceinline__ void settle(const DecodeParams& p, WaveState_<D>& ws, int64_t C, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (ws.pend[i].state == 2) resolve_piece<D>(p, ws.pend[i], C, lane);
  if (ws.pend[0].state == 1 || ws.pend[1].state == 1) {
    wait_vmcnt<LOADS>();
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (ws.pend[i].state == 1) count_piece(p, ws.pend[i], lane);
  }
}

template <int D, bool FP8, int NSUB>
__global__ __launch_bounds__(kDecodeThreads, PA_DECODE_MIN_WAVES) void decode_kernel(const DecodeParams p) {
  using Buf = StageBuf<D, FP8, NSUB>;
  static_assert(Buf::kLoads <= 63, "a stage must fit the vector-memory counter");
  const int lane = threadIdx.x & 63;
  // Workgroups are dispatched round-robin over the 8 XCDs; the ones that
  // start together take neighbouring ranges of one contiguous slice per
  // XCD.  The wavefront index is uniform across the wavefront; saying so
  // lets the compiler keep all per-wavefront control in scalar registers.
  const int ngroups = (p.num_waves + kWavesPerGroup - 1) / kWavesPerGroup;
  const int full = ngroups / 64 * 64;
  int g = blockIdx.x;
  if (g < full) g = (g / 64) * 64 + (g % 8) * 8 + (g % 64) / 8;
  const int wave = __builtin_amdgcn_readfirstlane(g * kWavesPerGroup + (threadIdx.x >> 6));
  if (wave >= p.num_waves) return;
  const int S = p.num_seqs, Hkv = p.num_kv_heads;
  const int max_len = p.max_blocks * p.block_size;

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
    total += uni(wave_reduce_sum(n));
  }
  const int64_t W = uni64(total * Hkv);
  int64_t C = p.chunk_fixed;
  if (C <= 0) {
    C = (W + p.num_waves - 1) / p.num_waves;
    if (C < p.chunk_min) C = p.chunk_min;
  }
  C = uni64(C);
  const int64_t a = uni64((int64_t)wave * C);
  if (a >= W) return;

  const int64_t b = (a + C < W) ? a + C : W;

  // Pass 2: the sequences holding chunks a and b - 1.
  Pos pa_, pz;
  pa_.s = pz.s = 0;
  pa_.before = pz.before = 0;
  {
    int64_t carry = 0;
    bool found_a = false, found_z = false;
    for (int base = 0; base < S && !(found_a && found_z); base += 64) {
      const int si = base + lane;
      int n = 0;
      if (si < S) n = chunks_of(p.seq_lens[si], max_len);
      n = n < 0 ? 0 : n;
      const int incl = wave_incl_scan(n, lane);
      const int64_t lo = (int64_t)Hkv * (carry + incl - n), hi = (int64_t)Hkv * (carry + incl);
      const uint64_t hit_a = __ballot(n > 0 && lo <= a && a < hi);
      const uint64_t hit_z = __ballot(n > 0 && lo <= b - 1 && b - 1 < hi);
      if (hit_a && !found_a) {
        const int l0 = uni(__builtin_ctzll(hit_a));
        pa_.s = uni(base + l0);
        pa_.before = uni64(carry + readlane(incl - n, l0));
        found_a = true;
      }
      if (hit_z && !found_z) {
        const int l0 = uni(__builtin_ctzll(hit_z));
        pz.s = uni(base + l0);
        pz.before = uni64(carry + readlane(incl - n, l0));
        found_z = true;
      }
      carry += readlane(incl, 63);
    }
  }
  Cursor cur;
  cur.a = a;
  cur.nq = 0;
  cur.new_piece = true;
  pa_.L = sload(p.seq_lens, pa_.s);
  pa_.n = chunks_of(pa_.L, max_len);
  pz.L = sload(p.seq_lens, pz.s);
  pz.n = chunks_of(pz.L, max_len);
  {
    const int64_t off = a - (int64_t)Hkv * pa_.before;
    pa_.h = uni((int)(off / pa_.n));
    pa_.j = uni((int)(off - (int64_t)pa_.h * pa_.n));
    pa_.x = a;
  }
  {
    const int64_t off = (b - 1) - (int64_t)Hkv * pz.before;
    pz.h = uni((int)(off / pz.n));
    pz.j = 0;  // walk the last piece from its unit's start (or from a)
    pz.x = (int64_t)Hkv * pz.before + (int64_t)pz.h * pz.n;
  }
  const int64_t a_unit_end = (int64_t)Hkv * pa_.before + (int64_t)(pa_.h + 1) * pa_.n;
  if (b <= a_unit_end) {
    // The whole range lies in one unit.
    pa_.end = b;
    cur.cur = pa_;
  } else {
    Pos mid = pa_;
    pa_.end = a_unit_end;
    pz.end = b;
    cur.cur = pa_;
    cur.queue[0] = pz;
    cur.nq = 1;
    if (a_unit_end < pz.x) {
      next_unit(mid, p, max_len);
      mid.x = a_unit_end;
      mid.end = pz.x;
      cur.queue[1] = mid;
      cur.nq = 2;
    }
  }

  // Two-stage software pipeline: the loads of the next stage are in flight
  // while the current stage's math runs.
  WaveState<D, FP8> ws;
  ws.pend[0].state = ws.pend[1].state = 0;
  ws.bad = false;
  Buf A, B;
  Stage sa = next_stage<NSUB>(cur, p, max_len);
  issue_stage<D, FP8, NSUB>(p, sa, A, lane);
  for (;;) {
    Stage sb = next_stage<NSUB>(cur, p, max_len);
    issue_stage<D, FP8, NSUB>(p, sb, B, lane);
    settle<D, Buf::kLoads>(p, ws, C, lane);
    finish_stage<D, FP8, NSUB>(p, sa, A, ws, wave, C, lane);
    if (!sb.valid) break;
    sa = next_stage<NSUB>(cur, p, max_len);
    issue_stage<D, FP8, NSUB>(p, sa, A, lane);
    settle<D, Buf::kLoads>(p, ws, C, lane);
    finish_stage<D, FP8, NSUB>(p, sb, B, ws, wave, C, lane);
    if (!sa.valid) break;
  }
  // Drain: everything issued has completed after this wait.
  wait_vmcnt<0>();
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (ws.pend[i].state == 2) resolve_piece<D>(p, ws.pend[i], C, lane);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (ws.pend[i].state == 1) {
      count_piece(p, ws.pend[i], lane);
      resolve_piece<D>(p, ws.pend[i], C, lane);
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
