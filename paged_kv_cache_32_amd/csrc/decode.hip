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
//    gives lane (d%16, t-group) 4 consecutive tokens of R dims 16 apart.
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (rows = tokens, cols = query
//    heads, fp32 accumulate; bf16 products are exact).  O^T = V^T P^T with
//    v_mfma_f32_16x16x16_bf16; P is split into a bf16 high part and a bf16
//    remainder so the probabilities keep ~16 significant bits.  fp8 codes
//    are widened to bf16 exactly on load.
//  * Online softmax in base 2 (scale * log2 e folded into the logit scale);
//    the accumulator is rescaled only when a head's maximum grows by more
//    than kRescaleSlack.
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
//  * Fused append (the APPEND instantiation): the step's new token of a
//    sequence is its position L - 1, in the last chunk of each of its units.
//    Before its first tile load, a wavefront stores the new tokens of the
//    units whose last chunk lies in its range (it is the only reader of
//    those tiles), 8 units per memory round trip, and waits for the stores;
//    its loads then read them like any other token.  All of the append's memory traffic thus happens
//    before the load pipeline starts: a load or store issued inside the
//    pipeline on some stages only would make the waits of the following
//    stages cover it, and under full load each such wait costs about one
//    memory latency.
#include "pa_internal.h"

// Sub-blocks loaded per online-softmax step, and the fewest wavefronts per
// SIMD the register allocation must leave room for.
#ifndef PA_DECODE_STAGE
#define PA_DECODE_STAGE 1
#endif
#ifndef PA_DECODE_STAGE_FP8
#define PA_DECODE_STAGE_FP8 4
#endif
#ifndef PA_DECODE_MIN_WAVES
#define PA_DECODE_MIN_WAVES 1
#endif
// 1: K/V tiles are read with the non-temporal hint (read once, no reuse).
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif
// Pieces whose partial records the merging wavefront loads per round trip.
#ifndef PA_DECODE_MERGE_BATCH
#define PA_DECODE_MERGE_BATCH 8
#endif

namespace pa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

// Largest growth of a query head's running maximum (base-2 logits) that is
// absorbed without rescaling: probabilities are then taken against the old
// maximum and may reach 2^kRescaleSlack, which the bf16 hi/lo operands and
// the fp32 sums carry as well as any other value.  The accumulator is
// rescaled only when some head's maximum grows by more, which after the
// first stage of a piece is rare.
constexpr float kRescaleSlack = 8.0f;

// Inclusive prefix sum over the wavefront's 64 lanes with DPP row shifts and
// row broadcasts (seven dependent VALU adds, no LDS permutes): each lane first
// sums itself and the three lanes before it in its row of 16, then the row
// sums double across banks (shift 4, then 8), and rows take the last lane of
// the row before them (broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_incl_scan(int v, int /*lane*/) {
  const int o = v;
  v += __builtin_amdgcn_update_dpp(0, o, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, o, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, o, 0x113, 0xf, 0xf, true);   // row_shr:3
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xe, true);   // row_shr:4, banks 1-3
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xc, true);   // row_shr:8, banks 2-3
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return v;
}

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// Sum over the wavefront, the same in every lane.
__device__ __forceinline__ int wave_reduce_sum(int v) { return readlane(wave_incl_scan(v, 0), 63); }

// First token a sequence of L tokens attends to: L - W with a window of W
// tokens ("KV Cache Engineering for LLM Serving", section 3, sliding
// windows), 0 without one (W = 0) or while L <= W.
__device__ __forceinline__ int window_lo(int L, int W) { return (W > 0 && L > W) ? L - W : 0; }

// Chunks (16-token pieces) of a sequence's unit: the chunks holding tokens
// [window_lo, L); -1 marks an invalid length.
__device__ __forceinline__ int chunks_of(int L, int max_len, int W) {
  if (L < 0 || L > max_len) return -1;
  return (L + kSub - 1) / kSub - window_lo(L, W) / kSub;
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
__device__ __forceinline__ void split_p(const float p[4], u32x2& hi, u32x2& lo) {
  uint32_t l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = __float_as_uint(p[i]);
    l[i] = __float_as_uint(p[i] - __uint_as_float(b & 0xFFFF0000u));
  }
  hi[0] = (__float_as_uint(p[0]) >> 16) | (__float_as_uint(p[1]) & 0xFFFF0000u);
  hi[1] = (__float_as_uint(p[2]) >> 16) | (__float_as_uint(p[3]) & 0xFFFF0000u);
  lo[0] = (l[0] >> 16) | (l[1] & 0xFFFF0000u);
  lo[1] = (l[2] >> 16) | (l[3] & 0xFFFF0000u);
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
  static constexpr int DC = D / 16;                 // 16-row blocks of O^T
  static constexpr int R = FP8 ? 4 : 2;             // dim blocks fed by one 16-byte V load
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
  float m;        // reference maximum of base-2 logits of query head (lane & 15)
  float l;        // this lane's share of the running sum
  f32x4 acc[D / 16];
};

// Stage flags.
enum : int {
  kValid = 1,    // the stage holds chunks
  kFirst = 2,    // first stage of a piece: load Q, reset the softmax state
  kLast = 4,     // last stage of a piece: write it out or store the partial
  kTail = 8,     // ends in the unit's last chunk, which is partial
  kAtA = 16,     // the piece starts at the wavefront's first chunk
  kWhole = 32,   // the piece is its whole unit
  kHead = 64,    // starts at the unit's first chunk, which begins before the window
};

// A piece: chunks [j0, j1) of unit (s, h), whose first chunk sits at u0 in
// the linear chunk list; the unit has n chunks and the sequence L tokens.
// Unit chunk j is the sequence's chunk window_lo(L, W) / 16 + j.  uw: the
// unit's first chunk in the weighted list that the split cuts (each unit
// preceded by its charge), set for the boundary pieces A and Z only, the
// only ones that can be part of a unit.
struct Piece {
  int s, h, n, L, u0, j0, j1, uw;
};

// One stage, uniform across the wavefront: chunks [j, j + cnt) of a piece,
// j counted in the sequence (not in the unit).
struct Stage {
  int s, h, n, L, u0, j, cnt, flags, uw;
};

// Where a wavefront stands in its range [a, b) of the chunk list.  The
// range is walked as the piece holding chunk a (A), then the piece holding
// chunk b - 1 (Z) when that is another unit, then the whole units between
// them: the boundary pieces, which other wavefronts share, go first so that
// split units are merged early rather than at the end of the kernel.
struct Cursor {
  Piece cur;       // piece being walked
  Piece z;         // piece Z (j1 = 0 when there is none; z.u0 ends the middle walk)
  int j;           // next chunk of cur
  int phase;       // 0: A, 1: Z, 2: middle units, 3: done
  int a_end;       // chunk-list index just past unit A
  int a_s, a_h;    // unit A, where the middle walk starts from
};

// A partial piece on its way to being counted in: stored (its stores must
// complete first), then counted (the counter's old value is in flight).
struct Pending {
  int state;       // 0 empty/done, 1 stored, 2 counted, 3 unit to be merged here, 4 group to be
                   // merged here
  int lvl;         // counted on: 1 its group's counter, 0 the unit's
  int s, h, u0, n, uw;
  int prior;       // lane 0: counter value before this piece was counted
};

// The unit after (s, h): (s, h + 1), or head 0 of the next sequence with
// chunks (n and L are updated then).  Only called while chunks remain, so
// such a sequence exists.
__device__ __forceinline__ void next_unit(const DecodeParams& p, int max_len, int& s, int& h,
                                          int& n, int& L) {
  if (h + 1 < p.num_kv_heads) {
    ++h;
    return;
  }
  h = 0;
  for (;;) {
    ++s;
    L = sload(p.seq_lens, s);
    n = chunks_of(L, max_len, p.window);
    if (n > 0) break;
  }
}

// Fused append: store the new tokens of up to 8 units at once, unit g by the
// 8 lanes 8g .. 8g + 7 (u_s >= 0 marks a lane whose group has a unit): the
// token of sequence u_s (position u_L - 1) of KV head u_h, rows [u_s][u_h][:]
// of k_new / v_new, goes into its tile as the cache write stores it (bf16
// bits, or e4m3fn codes of x / scale).  Lane j writes K pieces j and j + 8 of
// the row (16 bytes, X dims each) and V dims (D / 8) j .. + D / 8 - 1 one
// element each.  Every load of the batch is issued before the first store,
// so the batch costs one memory round trip.  Nothing is written for a token
// whose block lies outside the pool.  The stores carry the non-temporal hint
// (K pieces: [d/X][t%16][X]): they touch 48 lines per unit in part, and kept
// in L2 as partly written lines while the decode streams 1.3 GB past them
// they cost the 70B batch-64 layer 14 us, against under 3 us with the hint.
template <int D, bool FP8>
__device__ __forceinline__ void write_new_tokens(const DecodeParams& p, int u_s, int u_h, int u_L, int lane) {
  using T = Tile<D, FP8>;
  constexpr int X = FP8 ? 16 : 8;    // elements per 16-byte K piece
  constexpr int KP = D / X;          // K pieces per row
  constexpr int VE = D / 8;          // V elements per lane
  if (u_s < 0) return;
  const int j = lane & 7;
  const int pos = u_L - 1, chunk = pos / kSub, r = pos % kSub;
  const int bi = pos / p.block_size;
  const int blk = p.block_tables[(int64_t)u_s * p.max_blocks + (p.ring ? bi % p.max_blocks : bi)];
  const int64_t row = ((int64_t)u_s * p.num_kv_heads + u_h) * D;
  u32x4 kin[2][FP8 ? 2 : 1];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int hf = 0; hf < (FP8 ? 2 : 1); ++hf)
      kin[i][hf] = (j + 8 * i < KP) ? *reinterpret_cast<const u32x4*>(p.k_new + row + (j + 8 * i) * X + 8 * hf)
                                    : u32x4{0u, 0u, 0u, 0u};
  u32x4 vin[VE / 8];
#pragma unroll
  for (int i = 0; i < VE / 8; ++i) vin[i] = *reinterpret_cast<const u32x4*>(p.v_new + row + VE * j + 8 * i);
  if ((unsigned)blk >= (unsigned)p.num_blocks) return;
  const int64_t tile = (int64_t)blk * p.blk_stride + (int64_t)(u_h * p.subs + (chunk - bi * p.subs)) * T::TILE_BYTES;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int pc = j + 8 * i;
    if (pc < KP) {
      u32x4 out;
      if constexpr (FP8) {
        out = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t w = kin[i][e >> 3][(e >> 1) & 3];
          out[e >> 2] |= e4m3_code(bf16_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu)), p.k_inv) << (8 * (e & 3));
        }
      } else {
        out = kin[i][0];
      }
      __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(p.k_store + tile + ((int64_t)pc * kSub + r) * 16));
    }
  }
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    const uint32_t w = vin[e >> 3][(e >> 1) & 3];
    const uint32_t x = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
    const int d = VE * j + e;
    if constexpr (FP8)
      __builtin_nontemporal_store((uint8_t)e4m3_code(bf16_to_f32(x), p.v_inv), p.v_store + tile + v_elem<4>(d, r));
    else
      __builtin_nontemporal_store((uint16_t)x, reinterpret_cast<uint16_t*>(p.v_store + tile) + v_elem<2>(d, r));
  }
}

// Next stage of the cursor's range; moves the cursor past it.
template <int NSUB>
__device__ __forceinline__ Stage next_stage(Cursor& c, const DecodeParams& p, int max_len) {
  if (c.phase < 3 && c.j == c.cur.j1) {
    if (c.phase == 0 && c.z.j1 > 0) {
      c.cur = c.z;
      c.phase = 1;
    } else if (c.phase <= 1 && c.a_end < c.z.u0) {
      // First middle unit: the one after unit A.
      int s = c.a_s, h = c.a_h;
      int L = sload(p.seq_lens, s);
      int n = chunks_of(L, max_len, p.window);
      next_unit(p, max_len, s, h, n, L);
      c.cur = Piece{s, h, n, L, c.a_end, 0, n, 0};
      c.phase = 2;
    } else if (c.phase == 2 && c.cur.u0 + c.cur.n < c.z.u0) {
      int s = c.cur.s, h = c.cur.h, n = c.cur.n, L = c.cur.L;
      const int u0 = c.cur.u0 + n;
      next_unit(p, max_len, s, h, n, L);
      c.cur = Piece{s, h, n, L, u0, 0, n, 0};
    } else {
      c.phase = 3;
    }
    c.j = c.cur.j0;
  }
  Stage st;
  if (c.phase == 3) {
    st = Stage{0, 0, 0, 0, 0, 0, 0, 0, 0};
    return st;
  }
  const Piece& pc = c.cur;
  const int lo = window_lo(pc.L, p.window);
  const int c0 = lo / kSub;
  int cnt = pc.j1 - c.j;
  if (cnt > NSUB) cnt = NSUB;
  int f = kValid;
  if (c.j == pc.j0) f |= kFirst;
  if (c.j + cnt == pc.j1) f |= kLast;
  if (c.j + cnt == pc.n && (c0 + pc.n) * kSub > pc.L) f |= kTail;
  if (c.j == 0 && lo > c0 * kSub) f |= kHead;
  if (c.phase == 0) f |= kAtA;
  if (pc.j0 == 0 && pc.j1 == pc.n) f |= kWhole;
  st = Stage{uni(pc.s), uni(pc.h), uni(pc.n), uni(pc.L), uni(pc.u0), uni(c0 + c.j), uni(cnt), uni(f), uni(pc.uw)};
  c.j += cnt;
  return st;
}

// Fused append: store the new tokens of the units whose last chunk lies in
// this wavefront's range [a, b) (called before the first stage, while the
// cursor still stands at piece A), 8 units per batch, then wait for the
// stores.  Those units are unit A when it ends inside the range, every
// middle unit, and unit Z when its last chunk is b - 1.
template <int D, bool FP8>
__device__ __forceinline__ void append_range(const DecodeParams& p, const Cursor& c, int b, int max_len,
                                             int lane) {
  int u_s = -1, u_h = 0, u_L = 0, cnt = 0;
  auto add = [&](int s, int h, int L) {
    if ((lane >> 3) == cnt) {
      u_s = s;
      u_h = h;
      u_L = L;
    }
    if (++cnt == 8) {
      write_new_tokens<D, FP8>(p, u_s, u_h, u_L, lane);
      u_s = -1;
      cnt = 0;
    }
  };
  if (c.a_end <= b) add(c.cur.s, c.cur.h, c.cur.L);
  if (c.a_end < c.z.u0) {
    int s = c.a_s, h = c.a_h, n = c.cur.n, L = c.cur.L;
    int u0 = c.a_end;
    do {
      next_unit(p, max_len, s, h, n, L);
      add(s, h, L);
      u0 += n;
    } while (u0 < c.z.u0);
  }
  if (c.z.j1 > 0 && c.z.u0 + c.z.n == b) add(c.z.s, c.z.h, c.z.L);
  if (cnt > 0) write_new_tokens<D, FP8>(p, u_s, u_h, u_L, lane);
  wait_vmcnt<0>();
}

// Issue every load of a stage: exactly StageBuf::kLoads vector loads, always,
// so the wait counts the compiler derives do not depend on the branch taken.
// Chunk slots past the stage, tiles of out-of-pool blocks and the query of a
// stage that does not start a piece read tile 0 / query row 0 instead, with
// the same lane offsets, so every address stays inside its buffer.  Returns
// whether a block id of the stage lies outside the pool.
template <int D, bool FP8, int NSUB>
__device__ __forceinline__ bool issue_stage(const DecodeParams& p, const Stage& st,
                                            StageBuf<D, FP8, NSUB>& buf, int q_off, int k_off,
                                            int v_off) {
  using T = Tile<D, FP8>;
  const int G = p.group;
  // Query operand: lane (col = head in group, qd = k-group) holds 8 dims;
  // bf16 K tiles put dims 32c + 8qd .. +7 in MFMA c; fp8 K tiles put dims
  // 64(c/2) + 16qd + 8(c%2) .. +7 there.
  {
    const int64_t row = (st.flags & kFirst) ? ((int64_t)st.s * p.num_q_heads + (int64_t)st.h * G) * D : 0;
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(p.q + row) + q_off;
#pragma unroll
    for (int c = 0; c < T::QK; ++c) {
      const int imm = FP8 ? 128 * (c >> 1) + 16 * (c & 1) : 64 * c;
      buf.q[c] = *reinterpret_cast<const u32x4*>(qb + imm);
    }
  }
  // Block ids of the stage's chunks: chunk j lies in block j / subs at
  // sub-block j % subs.  All ids are loaded first (scalar loads); ids past
  // the stage repeat its last one, so no table entry past the sequence's
  // blocks is read.  With ring rows, logical block b sits at entry
  // b % max_blocks: a stage's blocks all lie in the window's span, fewer
  // than max_blocks consecutive blocks, so they wrap at most once.
  const int subs = p.subs;
  const int jlast = st.j + (st.cnt > 0 ? st.cnt - 1 : 0);
  const int bi0 = (subs == 1) ? st.j : (int)__umulhi((unsigned)st.j, p.subs_magic);
  const int bil = (subs == 1) ? jlast : (int)__umulhi((unsigned)jlast, p.subs_magic);
  const int32_t* bt = p.block_tables + (int64_t)st.s * p.max_blocks;
  const int e0 = p.ring ? uni(bi0 % p.max_blocks) : bi0;   // entry of block bi0
  int blk[NSUB], sub[NSUB];
  {
    int bi = bi0, sb = st.j - bi0 * subs;
#pragma unroll
    for (int k = 0; k < NSUB; ++k) {
      int e = e0 + ((bi < bil ? bi : bil) - bi0);
      if (e >= p.max_blocks) e -= p.max_blocks;
      blk[k] = sload(bt, e);
      sub[k] = sb;
      if (++sb == subs) {
        sb = 0;
        ++bi;
      }
    }
  }
  // KV head of the stage's tiles: the unit's head, or, with one head per
  // sequence (per-head block tables), sequence s's head s % seq_heads.
  int kvh = st.h;
  if (p.seq_heads > 1) kvh = uni(st.s - (int)__umulhi((unsigned)st.s, p.seq_heads_magic) * p.seq_heads);
  bool bad = false;
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    const bool in = k < st.cnt;
    const bool ok = (unsigned)blk[k] < (unsigned)p.num_blocks;
    bad |= in && !ok;
    const int64_t tile = (in && ok) ? (int64_t)blk[k] * p.blk_stride +
                                          (int64_t)(kvh * subs + sub[k]) * T::TILE_BYTES
                                    : 0;
    const uint8_t* kt = p.k_cache + tile + k_off;
    const uint8_t* vt = p.v_cache + tile + v_off;
#pragma unroll
    for (int c = 0; c < T::KLD; ++c) buf.k[k][c] = load_kv(reinterpret_cast<const u32x4*>(kt + c * 1024));
#pragma unroll
    for (int e = 0; e < T::VLD; ++e) buf.v[k][e] = load_kv(reinterpret_cast<const u32x4*>(vt + e * 1024));
  }
  return bad;
}

// bf16 pair {tokens 4qd, 4qd+1}, {4qd+2, 4qd+3} of sub-block k for the V^T
// operand rows 16 dc + col.
template <int D, bool FP8, int NSUB>
__device__ __forceinline__ u32x2 v_operand(const StageBuf<D, FP8, NSUB>& buf, int k, int dc) {
  using T = Tile<D, FP8>;
  u32x2 a;
  if constexpr (FP8) {
    const uint32_t w = buf.v[k][dc / T::R][dc % T::R];
    a[0] = fp8x2_to_bf16x2<false>(w);
    a[1] = fp8x2_to_bf16x2<true>(w);
  } else {
    a[0] = buf.v[k][dc / T::R][2 * (dc % T::R)];
    a[1] = buf.v[k][dc / T::R][2 * (dc % T::R) + 1];
  }
  return a;
}

// The math of one stage: logits, online-softmax update, P V accumulation.
// MASK: the stage holds a partial chunk (the unit's last, or its first when
// the window starts inside it), so logits of tokens outside [lo, L) are set
// to -inf and their V elements to zero (they hold arbitrary bits, possibly
// NaN, and 0 * NaN is NaN).
template <int D, bool FP8, int NSUB, bool MASK>
__device__ __forceinline__ void compute_stage(const DecodeParams& p, const Stage& st,
                                              const StageBuf<D, FP8, NSUB>& buf,
                                              const bf16x8* qop, Softmax<D>& sm, int lane) {
  using T = Tile<D, FP8>;
  const int qd = lane >> 4;
  const int first_tok = st.j * kSub;
  const int L = st.L;
  const int lo = MASK ? window_lo(L, p.window) : 0;

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
        z[k][i] = s[i] * p.qk_scale;
        if (MASK && (tok0 + i >= L || tok0 + i < lo)) z[k][i] = kNegInf;
        mx = __builtin_fmaxf(mx, z[k][i]);
      }
    }
  }
  mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (__builtin_amdgcn_ballot_w64(mx > sm.m + kRescaleSlack) != 0) {
    const float m_new = __builtin_fmaxf(sm.m, mx);
    const float alpha = (sm.m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(sm.m - m_new);
    sm.m = m_new;
    sm.l *= alpha;
#pragma unroll
    for (int dc = 0; dc < T::DC; ++dc) sm.acc[dc] *= alpha;
  }

  // O^T += V^T P^T, one 16-deep product per sub-block and P half; the V^T
  // operand of dim block dc is a register pair of the loaded tile, so the
  // loads feed the matrix cores without any register copies.
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    if (k < st.cnt) {
      float pz[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pz[i] = __builtin_amdgcn_exp2f(z[k][i] - sm.m);
      sm.l += (pz[0] + pz[1]) + (pz[2] + pz[3]);
      u32x2 p_hi, p_lo;
      split_p(pz, p_hi, p_lo);
      uint32_t m0 = 0xFFFFFFFFu, m1 = 0xFFFFFFFFu;
      if (MASK) {
        const int tok0 = first_tok + k * kSub + qd * 4;
        const bool t0 = tok0 + 0 < L && tok0 + 0 >= lo, t1 = tok0 + 1 < L && tok0 + 1 >= lo;
        const bool t2 = tok0 + 2 < L && tok0 + 2 >= lo, t3 = tok0 + 3 < L && tok0 + 3 >= lo;
        m0 = (t0 ? 0x0000FFFFu : 0u) | (t1 ? 0xFFFF0000u : 0u);
        m1 = (t2 ? 0x0000FFFFu : 0u) | (t3 ? 0xFFFF0000u : 0u);
      }
#pragma unroll
      for (int dc = 0; dc < T::DC; ++dc) {
        u32x2 a = v_operand<D, FP8, NSUB>(buf, k, dc);
        if (MASK) {
          a[0] &= m0;
          a[1] &= m1;
        }
        const i16x4 av = as_i16x4(a);
        sm.acc[dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, as_i16x4(p_hi), sm.acc[dc], 0, 0, 0);
        sm.acc[dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, as_i16x4(p_lo), sm.acc[dc], 0, 0, 0);
      }
    }
  }
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

// Pieces of wavefront w are stored in slot 2w (the piece that starts at the
// wavefront's first chunk) or 2w + 1 (the piece that ends at its last).
// Wavefront w covers the weighted positions [w C, (w + 1) C); a unit's piece
// in its first wavefront w0 is that wavefront's second piece when the chunk
// before the unit (weight uw - 1 - charge) lies in the same range.
__device__ __forceinline__ int piece_slot(int w, int w0, bool second) {
  return (w == w0 && second) ? 2 * w + 1 : 2 * w;
}

// Where a split unit's pieces are: wavefronts w0..w1, one piece each.  A
// unit of more than kTreeMinPieces pieces is merged as a tree when the
// workspace has group counters: the last piece counted in of each group of
// kMergeGroup consecutive pieces merges its group into the record slot of
// the group's first piece, and the last group counted in merges the group
// records.  The group merges run on many wavefronts at once, as their
// groups complete, so the unit's last merge reads a handful of group
// records instead of every piece (a unit of a long sequence split over a
// hundred wavefronts otherwise ends the launch with a long serial merge).
// Measured, the tree pays from 9 pieces on: with it only above 32 pieces
// the long-context batch (32 pieces per unit) took 342-345 us against
// 334-341 us.
constexpr int kMergeGroup = PA_DECODE_MERGE_BATCH;
constexpr int kTreeMinPieces = kMergeGroup;
struct UnitShape {
  int w0, w1;
  bool second;     // the piece in wavefront w0 is that wavefront's second piece
  bool tree;
};
__device__ __forceinline__ UnitShape unit_shape(const DecodeParams& p, const Pending& pd, int C) {
  UnitShape u;
  u.w0 = pd.uw / C;
  u.w1 = (pd.uw + pd.n - 1) / C;
  u.second = pd.u0 > 0 && pd.uw - 1 - p.unit_charge >= u.w0 * C;
  u.tree = p.group_counters != nullptr && u.w1 - u.w0 + 1 > kTreeMinPieces;
  return u;
}

// Merge the partial softmax states held in the record slots of wavefronts
// wf, wf + step, .. <= wl (pieces, or with step kMergeGroup the group
// records) of unit (s, h): out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M)
// l_p, M = max_p m_p, taken one record at a time with a running maximum.
// The result goes to out (and lse) when dst_slot < 0, else into record slot
// dst_slot as a record of its own (acc = the weighted sum, m = M, l = the
// weight), with the same device-coherent stores as the pieces.  Lane l
// handles kIt adjacent 4-float groups of one query head's row per pass, so
// one load of a record's (m, l) serves all of them; the loads of kBatch
// records are issued together (one memory round trip per kBatch records).
template <int D, int kIt, int kBatch>
__device__ __forceinline__ void merge_records(const DecodeParams& p, const Pending& pd, const UnitShape& u,
                                              int wf, int wl, int step, int dst_slot, int lane) {
  const int G = p.group;
  const int groups = G * D / 4;
  const int rec_bytes = G * (D + 4) * 4;
  f32x4* o = reinterpret_cast<f32x4*>(p.out + ((int64_t)pd.s * p.num_q_heads + (int64_t)pd.h * G) * D);
  for (int e0 = 0; e0 < groups; e0 += 64 * kIt) {
    const int e_first = e0 + lane * kIt;
    const int g = e_first / (D / 4), d40 = e_first - g * (D / 4);
    const bool in = e_first < groups;
    float M = kNegInf, den = 0.f;
    f32x4 num[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) num[it] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int wb = wf; wb <= wl; wb += kBatch * step) {
      f32x4 ml[kBatch], acc[kBatch][kIt];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int w = (wb + b * step <= wl) ? wb + b * step : wb;
        const auto r = record_rsrc(p.partials + (int64_t)piece_slot(w, u.w0, u.second) * (rec_bytes / 4), rec_bytes);
        ml[b] = load_record(r, in ? (G * D + g * 4) * 4 : 0);
#pragma unroll
        for (int it = 0; it < kIt; ++it) acc[b][it] = load_record(r, in ? ((d40 + it) * G + g) * 16 : 0);
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (wb + b * step <= wl) {
          const float m_new = __builtin_fmaxf(M, ml[b][0]);
          const float a = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M - m_new);
          const float f = (ml[b][0] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ml[b][0] - m_new);
#pragma unroll
          for (int it = 0; it < kIt; ++it) num[it] = num[it] * a + acc[b][it] * f;
          den = den * a + ml[b][1] * f;
          M = m_new;
        }
      }
    }
    if (dst_slot < 0) {
#pragma unroll
      for (int it = 0; it < kIt; ++it)
        if (in) o[e_first + it] = num[it] * (p.out_scale / den);
      if (p.lse && in && d40 == 0)
        p.lse[(int64_t)pd.s * p.num_q_heads + (int64_t)pd.h * G + g] = M + __builtin_amdgcn_logf(den);
    } else {
      const auto r = record_rsrc(p.partials + (int64_t)dst_slot * (rec_bytes / 4), rec_bytes);
#pragma unroll
      for (int it = 0; it < kIt; ++it)
        if (in) store_record(r, ((d40 + it) * G + g) * 16, num[it]);
      if (in && d40 == 0) store_record(r, (G * D + g * 4) * 4, f32x4{M, den, 0.f, 0.f});
    }
  }
}

// Count a stored piece in (its stores have completed): on its group's
// counter when the unit is merged as a tree, else on the unit's.
__device__ __forceinline__ void count_piece(const DecodeParams& p, Pending& pd, int C, int wave, int lane) {
  const UnitShape u = unit_shape(p, pd, C);
  int32_t* counter = p.counters + (int64_t)pd.s * p.num_kv_heads + pd.h;
  pd.lvl = 0;
  if (u.tree) {
    const int g = (wave - u.w0) / kMergeGroup;
    counter = p.group_counters + piece_slot(u.w0 + g * kMergeGroup, u.w0, u.second);
    pd.lvl = 1;
  }
  pd.prior = 0;
  if (lane == 0) pd.prior = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  pd.state = 2;
}

// Read the counter's old value.  The wavefront that counted in the last
// piece of a group merges the group (state 4); the one that counted in the
// unit's last piece, or last group, merges the unit (state 3) and then
// re-arms the counter for the next call; the others are done.
__device__ __forceinline__ void resolve_piece(const DecodeParams& p, Pending& pd, int C, int wave) {
  const int prior = readlane(pd.prior, 0);
  const UnitShape u = unit_shape(p, pd, C);
  const int pieces = u.w1 - u.w0 + 1;
  if (pd.lvl == 1) {
    const int g = (wave - u.w0) / kMergeGroup;
    const int size = pieces - g * kMergeGroup < kMergeGroup ? pieces - g * kMergeGroup : kMergeGroup;
    pd.state = (prior == size - 1) ? 4 : 0;
  } else {
    const int items = u.tree ? (pieces + kMergeGroup - 1) / kMergeGroup : pieces;
    pd.state = (prior == items - 1) ? 3 : 0;
  }
}

// The merges this wavefront owes, at the end of its range: a group (state
// 4) is merged into its first piece's slot, its counter re-armed, and the
// group counted in on the unit's counter once the group record's stores
// have completed, which may leave the unit's merge to this wavefront too
// (state 3).  One call site of the merge keeps a single copy of its code.
template <int D>
__device__ __forceinline__ void merge_owed(const DecodeParams& p, Pending& pd, int C, int wave, int lane) {
  const UnitShape u = unit_shape(p, pd, C);
  while (pd.state >= 3) {
    const bool group = pd.state == 4;
    int wf = u.w0, wl = u.w1, step = u.tree ? kMergeGroup : 1, dst = -1;
    if (group) {
      wf = u.w0 + (wave - u.w0) / kMergeGroup * kMergeGroup;
      wl = wf + kMergeGroup - 1 < u.w1 ? wf + kMergeGroup - 1 : u.w1;
      step = 1;
      dst = piece_slot(wf, u.w0, u.second);
    }
    merge_records<D, D / 32, kMergeGroup>(p, pd, u, wf, wl, step, dst, lane);
    if (group) {
      wait_vmcnt<0>();
      if (lane == 0) {
        __hip_atomic_store(p.group_counters + dst, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        pd.prior = __hip_atomic_fetch_add(p.counters + (int64_t)pd.s * p.num_kv_heads + pd.h, 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
      }
      pd.lvl = 0;
      resolve_piece(p, pd, C, wave);
    } else {
      if (lane == 0)
        __hip_atomic_store(p.counters + (int64_t)pd.s * p.num_kv_heads + pd.h, 0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      pd.state = 0;
    }
  }
}

// Per-wavefront state carried across stages.
template <int D, bool FP8>
struct WaveState {
  Softmax<D> sm;
  bool bad;
  Pending pend[2];
  bf16x8 q[Tile<D, FP8>::QK];
};

// Math of a stage plus, at a piece boundary, the piece's output.
template <int D, bool FP8, int NSUB>
__device__ __forceinline__ void finish_stage(const DecodeParams& p, const Stage& st, bool st_bad,
                                             const StageBuf<D, FP8, NSUB>& buf,
                                             WaveState<D, FP8>& ws, int wave, int lane) {
  using T = Tile<D, FP8>;
  if (!(st.flags & kValid)) return;
  const int qd = lane >> 4, col = lane & 15;
  const int G = p.group;
  if (st.flags & kFirst) {
#pragma unroll
    for (int c = 0; c < T::QK; ++c) ws.q[c] = as_bf16x8(col < G ? buf.q[c] : u32x4{0u, 0u, 0u, 0u});
    ws.sm.m = kNegInf;
    ws.sm.l = 0.f;
#pragma unroll
    for (int dc = 0; dc < T::DC; ++dc) ws.sm.acc[dc] = f32x4{0.f, 0.f, 0.f, 0.f};
    ws.bad = false;
  }
  ws.bad |= st_bad;
  if (st.flags & (kTail | kHead))
    compute_stage<D, FP8, NSUB, true>(p, st, buf, ws.q, ws.sm, lane);
  else
    compute_stage<D, FP8, NSUB, false>(p, st, buf, ws.q, ws.sm, lane);
  if (!(st.flags & kLast)) return;

  float ltot = ws.sm.l + __shfl_xor(ws.sm.l, 16, 64);
  ltot += __shfl_xor(ltot, 32, 64);
  if (ws.bad) ltot = __builtin_nanf("");
  if (st.flags & kWhole) {
    // The whole unit is this wavefront's: write the output directly.
    if (col < G) {
      const float inv = p.out_scale / ltot;
      const int64_t row = (int64_t)st.s * p.num_q_heads + (int64_t)st.h * G + col;
      float* o = p.out + row * D + qd * 4;
#pragma unroll
      for (int dc = 0; dc < T::DC; ++dc) *reinterpret_cast<f32x4*>(o + dc * 16) = ws.sm.acc[dc] * inv;
      if (p.lse && qd == 0) p.lse[row] = ws.sm.m + __builtin_amdgcn_logf(ltot);
    }
    return;
  }
  const int slot = (st.flags & kAtA) ? 2 * wave : 2 * wave + 1;
  const int rec_bytes = G * (D + 4) * 4;
  const auto r = record_rsrc(p.partials + (int64_t)slot * (rec_bytes / 4), rec_bytes);
  if (col < G) {
#pragma unroll
    for (int dc = 0; dc < T::DC; ++dc) store_record(r, ((dc * 4 + qd) * G + col) * 16, ws.sm.acc[dc]);
    if (qd == 0) store_record(r, (G * D + col * 4) * 4, f32x4{ws.sm.m, ltot, 0.f, 0.f});
  }
  // A wavefront stores at most two pieces (its boundary pieces A and Z), so
  // a free slot always exists.
  Pending& pd = (ws.pend[0].state == 0) ? ws.pend[0] : ws.pend[1];
  pd.state = 1;
  pd.s = st.s;
  pd.h = st.h;
  pd.u0 = st.u0;
  pd.n = st.n;
  pd.uw = st.uw;
}

// Advance the pieces waiting to be counted in.  Called right after a
// stage's loads were issued: every piece stored before that issue has its
// stores complete once all but those loads are done, and every counter
// value read before it has arrived by then too.  A merge this wavefront
// owes is left for the end of its range, where the registers that hold the
// pipeline's loads are free for the merge's own.
template <int D, bool FP8, int LOADS>
__device__ __forceinline__ void settle(const DecodeParams& p, WaveState<D, FP8>& ws, int C, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (ws.pend[i].state == 2) resolve_piece(p, ws.pend[i], C, wave);
  if (ws.pend[0].state == 1 || ws.pend[1].state == 1) {
    wait_vmcnt<LOADS>();
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (ws.pend[i].state == 1) count_piece(p, ws.pend[i], C, wave, lane);
  }
}

template <int D, bool FP8, int NSUB, bool APPEND>
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
  const int wave = uni(g * kWavesPerGroup + (threadIdx.x >> 6));
  if (wave >= p.num_waves) return;
  const int S = p.num_seqs, Hkv = p.num_kv_heads;
  // Longest valid sequence: the table's reach, or with ring rows any length
  // whose chunk count stays inside int range.
  const int max_len = p.ring ? INT32_MAX - kSub : p.max_blocks * p.block_size;

  // Pass 1: total chunks and sequences with chunks.  Wavefront 0 also
  // writes the rows no other wavefront will touch: zeros for empty
  // sequences, NaN for invalid ones.
  int total = 0, filled = 0;
  for (int base = 0; base < S; base += 64) {
    const int si = base + lane;
    int n = 0;
    if (si < S) n = chunks_of(p.seq_lens[si], max_len, p.window);
    if (wave == 0) {
      uint64_t todo = __ballot(si < S && n <= 0);
      while (todo) {
        const int l0 = __builtin_ctzll(todo);
        todo &= todo - 1;
        const float v = (readlane(n, l0) < 0) ? __builtin_nanf("") : 0.f;
        float* o = p.out + (int64_t)(base + l0) * p.num_q_heads * D;
        for (int e = lane; e < p.num_q_heads * D / 4; e += 64)
          reinterpret_cast<f32x4*>(o)[e] = f32x4{v, v, v, v};
        if (p.lse)
          for (int e = lane; e < p.num_q_heads; e += 64)
            p.lse[(int64_t)(base + l0) * p.num_q_heads + e] = (v == 0.f) ? kNegInf : v;
      }
    }
    n = n < 0 ? 0 : n;
    total += uni(wave_reduce_sum(n));
    filled += uni(wave_reduce_sum(n > 0 ? 1 : 0));
  }
  // The host guarantees num_seqs * Hkv * (chunks per sequence) < 2^30, so
  // every chunk-list index below fits an int.
  //
  // The split cuts a weighted list: each unit (sequence, KV head) counts as
  // its chunks plus `charge` more in front of them, for the fixed costs a
  // unit brings to the wavefront that starts it (the sequence's length and
  // table entries, the query, a partial record).  Wavefront w takes the
  // weighted positions [w C, (w + 1) C), i.e. the chunks whose position (the
  // chunk's index plus the charges of its unit and the units before it)
  // falls there.  With no charge (fixed partitions) positions are chunk
  // indices.
  const int charge = p.unit_charge;
  const int W = uni(total * Hkv);
  const int Wt = uni(W + charge * Hkv * filled);
  int C = p.chunk_fixed;
  if (C <= 0) {
    C = (Wt + p.num_waves - 1) / p.num_waves;
    if (C < p.chunk_min) C = p.chunk_min;
  }
  C = uni(C);
  if ((int64_t)wave * C >= Wt) return;
  int a = uni(wave * C);
  int b = (Wt - a > C) ? a + C : Wt;
  if (charge > 0) {
    // The first chunk at or after weighted position a, and the one at or
    // after b (W when there is none).
    const int xa = a, xb = b;
    a = W;
    b = W;
    bool fa = false, fb = false;
    int carry_w = 0, carry_c = 0;
    for (int base = 0; base < S && !(fa && fb); base += 64) {
      const int si = base + lane;
      int n = 0;
      if (si < S) n = chunks_of(p.seq_lens[si], max_len, p.window);
      n = n < 0 ? 0 : n;
      const int span = n > 0 ? Hkv * (n + charge) : 0;
      const int incl_w = wave_incl_scan(span, lane);
      const int incl_c = wave_incl_scan(Hkv * n, lane);
      const int lo_w = carry_w + incl_w - span;
      const uint64_t hit_a = __ballot(n > 0 && lo_w <= xa && xa < lo_w + span);
      const uint64_t hit_b = __ballot(n > 0 && lo_w <= xb && xb < lo_w + span);
      if (hit_a && !fa) {
        const int l0 = uni(__builtin_ctzll(hit_a));
        const int nn = readlane(n, l0), rel = xa - readlane(lo_w, l0);
        const int h = rel / (nn + charge), off = rel - h * (nn + charge);
        a = uni(carry_c + readlane(incl_c, l0) - Hkv * nn + h * nn + (off < charge ? 0 : off - charge));
        fa = true;
      }
      if (hit_b && !fb) {
        const int l0 = uni(__builtin_ctzll(hit_b));
        const int nn = readlane(n, l0), rel = xb - readlane(lo_w, l0);
        const int h = rel / (nn + charge), off = rel - h * (nn + charge);
        b = uni(carry_c + readlane(incl_c, l0) - Hkv * nn + h * nn + (off < charge ? 0 : off - charge));
        fb = true;
      }
      carry_w += readlane(incl_w, 63);
      carry_c += readlane(incl_c, 63);
    }
    if (a >= b) return;     // a range inside one unit's charge (C > charge rules it out)
  }

  // Pass 2: the sequences holding chunks a and b - 1, the chunks of the
  // sequences before them, and how many of those have chunks.
  int sa = 0, sz = 0, before_a = 0, before_z = 0, filled_a = 0, filled_z = 0;
  {
    int carry = 0, carry_f = 0;
    bool found_a = false, found_z = false;
    for (int base = 0; base < S && !(found_a && found_z); base += 64) {
      const int si = base + lane;
      int n = 0;
      if (si < S) n = chunks_of(p.seq_lens[si], max_len, p.window);
      n = n < 0 ? 0 : n;
      const int incl = wave_incl_scan(n, lane);
      const int incl_f = wave_incl_scan(n > 0 ? 1 : 0, lane);
      const int lo = Hkv * (carry + incl - n), hi = Hkv * (carry + incl);
      const uint64_t hit_a = __ballot(n > 0 && lo <= a && a < hi);
      const uint64_t hit_z = __ballot(n > 0 && lo <= b - 1 && b - 1 < hi);
      if (hit_a && !found_a) {
        const int l0 = uni(__builtin_ctzll(hit_a));
        sa = uni(base + l0);
        before_a = uni(carry + readlane(incl - n, l0));
        filled_a = uni(carry_f + readlane(incl_f, l0) - 1);
        found_a = true;
      }
      if (hit_z && !found_z) {
        const int l0 = uni(__builtin_ctzll(hit_z));
        sz = uni(base + l0);
        before_z = uni(carry + readlane(incl - n, l0));
        filled_z = uni(carry_f + readlane(incl_f, l0) - 1);
        found_z = true;
      }
      carry += readlane(incl, 63);
      carry_f += readlane(incl_f, 63);
    }
  }
  Cursor cur;
  {
    const int La = sload(p.seq_lens, sa), na = chunks_of(La, max_len, p.window);
    const int ha = uni((a - Hkv * before_a) / na);
    const int u0a = Hkv * before_a + ha * na;
    const int a_end = u0a + na;
    // Weighted position of a unit's first chunk: its index plus the charges
    // of the units up to and including it.
    const int uwa = u0a + charge * (Hkv * filled_a + ha + 1);
    cur.cur = Piece{sa, ha, na, La, u0a, a - u0a, (b < a_end ? b : a_end) - u0a, uwa};
    cur.j = cur.cur.j0;
    cur.phase = 0;
    cur.a_end = a_end;
    cur.a_s = sa;
    cur.a_h = ha;
    cur.z = Piece{0, 0, 0, 0, a_end, 0, 0, 0};  // no piece Z: j1 = 0, middle walk ends at a_end
    if (b > a_end) {
      const int Lz = sload(p.seq_lens, sz), nz = chunks_of(Lz, max_len, p.window);
      const int hz = uni((b - 1 - Hkv * before_z) / nz);
      const int u0z = Hkv * before_z + hz * nz;
      cur.z = Piece{sz, hz, nz, Lz, u0z, 0, b - u0z, u0z + charge * (Hkv * filled_z + hz + 1)};
    }
  }
  if constexpr (APPEND) append_range<D, FP8>(p, cur, b, max_len, lane);

  // Lane offsets of the stage loads (constant per lane): query row of head
  // col (clamped into the group) at k-group qd; K lane = 16 bytes; V lane
  // (col, qd) reads tokens 4qd..4qd+3 of dims 16(R e + r) + col.
  const int qd = lane >> 4, col = lane & 15;
  const int q_off = ((col < p.group ? col : p.group - 1) * D) * 2 + (FP8 ? 32 : 16) * qd;
  const int k_off = lane * 16;
  const int v_off = (col * 4 + qd) * 16;

  // Two-stage software pipeline: the loads of the next stage are in flight
  // while the current stage's math runs.
  WaveState<D, FP8> ws;
  ws.pend[0].state = ws.pend[1].state = 0;
  ws.bad = false;
  Buf A, B;
  Stage sta = next_stage<NSUB>(cur, p, max_len);
  bool bad_a = issue_stage<D, FP8, NSUB>(p, sta, A, q_off, k_off, v_off);
  for (;;) {
    const Stage stb = next_stage<NSUB>(cur, p, max_len);
    const bool bad_b = issue_stage<D, FP8, NSUB>(p, stb, B, q_off, k_off, v_off);
    settle<D, FP8, Buf::kLoads>(p, ws, C, wave, lane);
    finish_stage<D, FP8, NSUB>(p, sta, bad_a, A, ws, wave, lane);
    if (!(stb.flags & kValid)) break;
    sta = next_stage<NSUB>(cur, p, max_len);
    bad_a = issue_stage<D, FP8, NSUB>(p, sta, A, q_off, k_off, v_off);
    settle<D, FP8, Buf::kLoads>(p, ws, C, wave, lane);
    finish_stage<D, FP8, NSUB>(p, stb, bad_b, B, ws, wave, lane);
    if (!(sta.flags & kValid)) break;
  }
  // Drain: everything issued has completed after this wait.
  wait_vmcnt<0>();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (ws.pend[i].state == 1) count_piece(p, ws.pend[i], C, wave, lane);
    if (ws.pend[i].state == 2) resolve_piece(p, ws.pend[i], C, wave);
    if (ws.pend[i].state >= 3) merge_owed<D>(p, ws.pend[i], C, wave, lane);
  }
}

// Sub-blocks per stage: one for bf16 (8 KiB of K and V per stage, two
// stages in flight), four for fp8 (16 KiB).  Measured on MI355X, one bf16
// sub-block per stage beat two by 1-2 % on long reads, and fp8 stages of
// two sub-blocks lost 7 % to four.
template <bool FP8>
constexpr int kStage = FP8 ? PA_DECODE_STAGE_FP8 : PA_DECODE_STAGE;

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

template <int D, bool FP8>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream) {
  const unsigned groups = (unsigned)((p.num_waves + kWavesPerGroup - 1) / kWavesPerGroup);
  if (p.k_new)
    hipLaunchKernelGGL((decode_kernel<D, FP8, kStage<FP8>, true>), dim3(groups), dim3(kDecodeThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<D, FP8, kStage<FP8>, false>), dim3(groups), dim3(kDecodeThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool FP8>
int resident_waves_typed() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<D, FP8, kStage<FP8>, false>, kDecodeThreads, 0) !=
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
