// Shared-prefix (cascade) decode: attention over the blocks a group of
// sequences shares is computed once per block for all of them.
//
// Sequences whose prompts start alike hold the same physical blocks for that
// prefix ("Taming the token torrent", "Implementing Radix Tree Prefix
// Caching"; "KV Cache Engineering for LLM Serving", section 11).  Softmax
// attention over a sequence's tokens splits at any token into parts whose
// partial states (m, l, acc) merge exactly by log-sum-exp, so a shared run
// of blocks (a segment) can be attended to for all of its member sequences
// in one pass over its K/V, and each sequence's remaining tokens by the
// ordinary paged decode; a last kernel merges the parts.
//
// segment_kernel: workgroup = (segment chunk, KV head h, up to
// PA_CASCADE_WAVES * MPW member sequences).  Each 16-token K/V tile of the
// chunk is loaded once into LDS, straight from global memory into one of
// three stage buffers, and used by all the workgroup's wavefronts; a
// wavefront holds MPW = 16 / G members' query groups as the 16 columns of
// its MFMA tiles (S^T = K Q^T and O^T = V^T P^T, both 16x16x32 bf16, P split
// into bf16 hi + lo), with the K operands in the paged decode's layout.
// Each (member, chunk) gets a partial record {acc[D], m, l} per query head
// of h.
//
// combine_kernel: per (sequence, query head, 4 dims), the private part's
// normalized output and log2-sum-exp from the decode kernel and the
// sequence's partial records, merged: out = sum_k 2^(lse_k - M) out_k /
// sum_k 2^(lse_k - M), lse_k = m_k + log2 l_k, out_k = acc_k / l_k.
#include "../../include/pa_cascade.h"
#include "pa_internal.h"

namespace pa {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kSlack = 8.0f;   // the running maximum is raised only when it grows by more
constexpr float kSlackWeight = 256.0f;   // 2^kSlack

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ i16x4 as_i16x4(u32x2 v) { return __builtin_bit_cast(i16x4, v); }

template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// hi = p truncated to bf16, lo = (p - hi) truncated to bf16; pairs packed
// with one byte permute each (the high halves of two words).
__device__ __forceinline__ uint32_t high_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ void split_p(const float p[4], u32x2& hi, u32x2& lo) {
  uint32_t l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = __float_as_uint(p[i]);
    l[i] = __float_as_uint(p[i] - __uint_as_float(b & 0xFFFF0000u));
  }
  hi[0] = high_halves(__float_as_uint(p[0]), __float_as_uint(p[1]));
  hi[1] = high_halves(__float_as_uint(p[2]), __float_as_uint(p[3]));
  lo[0] = high_halves(l[0], l[1]);
  lo[1] = high_halves(l[2], l[3]);
}

template <int D, bool FP8>
struct SegTile {
  static constexpr int EB = FP8 ? 1 : 2;
  static constexpr int BYTES = kSub * D * EB;        // one (block, head, sub-block) tile of K or of V
  static constexpr int KLD = FP8 ? D / 64 : D / 32;  // 16-byte K operand reads per lane and tile
  static constexpr int QK = D / 32;                  // 16x16x32 MFMAs per tile (K Q^T)
  static constexpr int DC = D / 16;                  // 16-row blocks of O^T
  static constexpr int R = FP8 ? 4 : 2;              // dim blocks per 16-byte V piece of the cache
  static constexpr int H = 16 / R;                   // O^T rows of one block that share a piece
  static constexpr int VLD = DC / R;                 // 1 KB blocks of a V tile
  static constexpr int PIECES = BYTES / 16;          // 16-byte pieces per tile
  static constexpr int TS = 8192 / BYTES;            // tiles per stage: 2, 4 or 8
  static constexpr int U = 16 / R;                   // bytes of 4 tokens of one dim
  static_assert(TS * VLD == PA_CASCADE_WAVES, "one V block per wavefront and stage");
};

constexpr int kSegThreads = 64 * PA_CASCADE_WAVES;
constexpr int kHalfStage = 8192;    // a stage: K tiles (8 KB) then V tiles (8 KB)
constexpr int kStages = 3;          // stage buffers in LDS: the one worked on and two loading
static_assert(kSegThreads * 16 == kHalfStage, "one K piece and one V piece per thread and stage");

// s_waitcnt immediate that waits until at most n vector memory operations
// of this wavefront are outstanding (expcnt and lgkmcnt left alone).
constexpr unsigned vmcnt_imm(unsigned n) { return (n & 15u) | (7u << 4) | (15u << 8) | ((n >> 4) << 14); }

// LDS image of a stage, filled by direct global-to-LDS loads of whole
// 16-byte pieces (each wavefront instruction writes 1 KB, lane L at 16 L).
// K tiles keep the cache layout: lane (token t, group g) reads the 8 (bf16)
// or 16 (fp8) consecutive dims of K operand c.  A V tile keeps its 1 KB
// blocks of R dim blocks, but each block's 64 pieces are reordered: the
// piece of dims 16 (R e + r) + dd (r = 0 .. R - 1), tokens 4 g .. 4 g + 3,
// goes to slot (dd / H) 4H + g H + dd % H.  O^T block j = R e + s takes on
// row m the dim 16 (R e + r) + dd with r = (m / H) ^ s, dd = m % H + H s,
// so its A operand for lane (m, g) is the 16 / R bytes of piece slot
// s 4H + g H + m % H at part r, from tile 2p then tile 2p + 1 (8 tokens of
// one dim), and the 16 lanes of a token group read 256 / R contiguous bytes.
template <int D, bool FP8>
__global__ __launch_bounds__(kSegThreads) void segment_kernel(const SegmentParams p) {
  using T = SegTile<D, FP8>;
  // Three separate arrays, so that the compiler sees that the loads into
  // one buffer do not touch the others and adds no waits for them.
  __shared__ __attribute__((aligned(16))) uint8_t lds0[2 * kHalfStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[2 * kHalfStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds2[2 * kHalfStage];
  static_assert(kStages == 3, "one array per stage buffer");
  auto stage_buf = [&](int j) -> uint8_t* { return j == 0 ? lds0 : j == 1 ? lds1 : lds2; };
  __shared__ int32_t ids[PA_CASCADE_MAX_CHUNK_BLOCKS];
  const int32_t* it = p.items + (int64_t)blockIdx.x * 8;
  const int blk_off = it[0], mem_off = it[2], nmem = it[3], h = it[4], slot0 = it[5];
  const int nblk = it[1] <= PA_CASCADE_MAX_CHUNK_BLOCKS ? it[1] : 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qd = lane >> 4, col = lane & 15;
  const int G = p.group, MPW = p.mpw;
  const int subs = p.block_size / kSub;
  const int ntiles = nblk * subs;
  const int nst = (ntiles + T::TS - 1) / T::TS;
  if ((unsigned)h >= (unsigned)(p.num_q_heads / G)) return;   // not a KV head: the item is skipped

  // This lane's column: member (wave * MPW + col / G) of the item, head col % G.
  const int mk = wave * MPW + col / G;
  const int seq = (col < MPW * G && mk < nmem) ? p.members[mem_off + mk] : -1;
  const bool col_ok = (unsigned)seq < (unsigned)p.num_seqs && (unsigned)(slot0 + mk) < (unsigned)p.num_slots;
  const int qh = h * G + col % G;
  bf16x8 qop[T::QK];
  {
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(p.q + ((int64_t)(col_ok ? seq : 0) * p.num_q_heads + qh) * D) +
                        (FP8 ? 32 : 16) * qd;
#pragma unroll
    for (int c = 0; c < T::QK; ++c) {
      const int imm = FP8 ? 128 * (c >> 1) + 16 * (c & 1) : 64 * c;
      const u32x4 v = *reinterpret_cast<const u32x4*>(qb + imm) ^ p.q_sign;
      qop[c] = as_bf16x8(col_ok ? v : u32x4{0u, 0u, 0u, 0u});
    }
  }

  // The chunk's block ids, once; a block id outside the pool reads tile 0
  // instead and marks the records NaN, as the paged decode marks such rows.
  bool bad = it[1] != nblk;
  for (int b = tid; b < nblk; b += kSegThreads) {
    const int blk = p.seg_blocks[blk_off + b];
    const bool ok = (unsigned)blk < (unsigned)p.num_blocks;
    bad |= !ok;
    ids[b] = ok ? blk : 0;
  }
  bad = __syncthreads_or(bad);
  // The query loads are complete before the stage loads start, so that no
  // later wait for them has to cover the stage loads as well.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // Per stage, thread tid brings K piece tid (tile tid / PIECES) to slot
  // tid, and wavefront w fills V block w % VLD of tile w / VLD, lane L
  // taking the piece its slot holds (see above).  Both tiles are the same
  // for a whole wavefront, so their addresses are scalar.
  const int kt = __builtin_amdgcn_readfirstlane(tid / T::PIECES);
  const uint32_t kpc = (tid % T::PIECES) * 16;
  const int vt = __builtin_amdgcn_readfirstlane(wave / T::VLD), ve = wave % T::VLD;
  uint32_t vpc;
  {
    const int s_ = lane / (4 * T::H), g_ = (lane / T::H) % 4, dd = lane % T::H + T::H * s_;
    vpc = (uint32_t)(((ve * 16 + dd) * 4 + g_) * 16);
  }
  const uint32_t magic = subs > 1 ? 0xFFFFFFFFu / (uint32_t)subs + 1u : 0u;   // t / subs for t < 2^16
  // Block ids of the two tiles of stage `stage` this wavefront brings.
  auto stage_ids = [&](int stage, int& tk, int& tv, int& bk, int& bv) {
    tk = stage * T::TS + kt;
    tk = tk < ntiles ? tk : ntiles - 1;               // past the end: a valid tile, never used
    tv = stage * T::TS + vt;
    tv = tv < ntiles ? tv : ntiles - 1;
    const int b0 = subs > 1 ? (int)__umulhi((uint32_t)tk, magic) : tk;
    const int b1 = subs > 1 ? (int)__umulhi((uint32_t)tv, magic) : tv;
    bk = __builtin_amdgcn_readfirstlane(ids[b0]);
    bv = __builtin_amdgcn_readfirstlane(ids[b1]);
    tk -= b0 * subs;
    tv -= b1 * subs;
  };
  // Both pieces of stage `stage` straight into LDS buffer `buf`.
  auto issue = [&](int stage, int buf) {
    int sk, sv, bk, bv;
    stage_ids(stage, sk, sv, bk, bv);
    const uint8_t* kb = p.k_cache + (int64_t)bk * p.blk_stride + (int64_t)(h * subs + sk) * T::BYTES;
    const uint8_t* vb = p.v_cache + (int64_t)bv * p.blk_stride + (int64_t)(h * subs + sv) * T::BYTES;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kb + kpc),
                                     (__attribute__((address_space(3))) void*)(stage_buf(buf) + wave * 1024), 16, 0,
                                     0);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vb + vpc),
                                     (__attribute__((address_space(3))) void*)(stage_buf(buf) + kHalfStage +
                                                                                wave * 1024),
                                     16, 0, 0);
  };

  float m = kNegInf, l = 0.f;
  f32x4 acc[T::DC];
#pragma unroll
  for (int dc = 0; dc < T::DC; ++dc) acc[dc] = f32x4{0.f, 0.f, 0.f, 0.f};

  // S^T = K Q^T of one tile from LDS.
  auto logits = [&](const uint8_t* kt_) -> f32x4 {
    // Each K operand is read one MFMA ahead of its use.
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
    u32x4 kn = *reinterpret_cast<const u32x4*>(kt_ + lane * 16);
#pragma unroll
    for (int c = 0; c < T::KLD; ++c) {
      const u32x4 kw = kn;
      if (c + 1 < T::KLD) kn = *reinterpret_cast<const u32x4*>(kt_ + (c + 1) * 1024 + lane * 16);
      if constexpr (FP8) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          u32x4 w;
          w[0] = fp8x2_to_bf16x2<false>(kw[2 * hf]);
          w[1] = fp8x2_to_bf16x2<true>(kw[2 * hf]);
          w[2] = fp8x2_to_bf16x2<false>(kw[2 * hf + 1]);
          w[3] = fp8x2_to_bf16x2<true>(kw[2 * hf + 1]);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w), qop[2 * c + hf], sc, 0, 0, 0);
        }
      } else {
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kw), qop[c], sc, 0, 0, 0);
      }
    }
    return sc;
  };

  // Lane part of the V operand reads: slot g H + m % H of block part s,
  // at byte (r = (m / H) ^ s) * U; one address per s.
  uint32_t voff[T::R];
#pragma unroll
  for (int s_ = 0; s_ < T::R; ++s_)
    voff[s_] = (uint32_t)((s_ * 4 * T::H + qd * T::H + col % T::H) * 16 + (((col / T::H) ^ s_) * T::U));

  // Tiles 2p and 2p + 1 of a stage (the second only when `two`): online
  // softmax in base 2 over the lane's 8 logits (tokens 4 qd + i of either
  // tile, column col), then O^T += V^T P^T with k slots 8 qd .. 8 qd + 7
  // pairing the A operand's 8 tokens with P split into bf16 hi and lo.
  // The weights are first taken against the running maximum m; one above
  // 2^kSlack (or infinite, while m is -inf) means some logit exceeds m by
  // more than kSlack, which a ballot decides: then the column's maximum of
  // the raw logits is taken (qk_scale >= 0, so it scales to the maximum of
  // the scaled ones), acc and l are rescaled and the weights taken again.
  // A missing second tile gets the exponent offset +inf, so weight 0.
  auto pair = [&](const uint8_t* buf, int pp, bool two) {
    const f32x4 s0 = logits(buf + 2 * pp * T::BYTES);
    const f32x4 s1 = logits(buf + (2 * pp + 1) * T::BYTES);
    const uint8_t* v0 = buf + kHalfStage + 2 * pp * T::BYTES;
    float pz[8];
    auto weights = [&]() {
      const float m1 = two ? m : __builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pz[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], p.qk_scale, -m));
        pz[4 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], p.qk_scale, -m1));
      }
    };
    weights();
    const float pmx = __builtin_fmaxf(
        __builtin_fmaxf(__builtin_fmaxf(pz[0], pz[1]), __builtin_fmaxf(pz[2], pz[3])),
        __builtin_fmaxf(__builtin_fmaxf(pz[4], pz[5]), __builtin_fmaxf(pz[6], pz[7])));
    if (__builtin_amdgcn_ballot_w64(pmx > kSlackWeight) != 0) {
      const float t1 = two ? __builtin_fmaxf(__builtin_fmaxf(s1[0], s1[1]), __builtin_fmaxf(s1[2], s1[3]))
                           : kNegInf;
      const float smx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(s0[0], s0[1]),
                                                         __builtin_fmaxf(s0[2], s0[3])), t1);
      const float lmx = smx * p.qk_scale;
      float mx = __builtin_fmaxf(lmx, __shfl_xor(lmx, 16, 64));
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = __builtin_fmaxf(m, mx);
      const float alpha = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dc = 0; dc < T::DC; ++dc) acc[dc] *= alpha;
      weights();
    }
    l += ((pz[0] + pz[1]) + (pz[2] + pz[3])) + ((pz[4] + pz[5]) + (pz[6] + pz[7]));
    u32x2 h0, l0, h1, l1;
    split_p(pz, h0, l0);
    split_p(pz + 4, h1, l1);
    const u32x4 bh = {h0[0], h0[1], h1[0], h1[1]}, bl = {l0[0], l0[1], l1[0], l1[1]};
    // V operand j, as the A operand of a 16x16x32 MFMA: 8 tokens (4 of tile
    // 2p, then 4 of tile 2p + 1) of one dim, widened to bf16 for fp8.
    auto v_op = [&](int j) -> u32x4 {
      const int off = (j / T::R) * 1024;
      u32x4 a;
      if constexpr (FP8) {
        const uint32_t w0 = *reinterpret_cast<const uint32_t*>(v0 + voff[j % T::R] + off);
        const uint32_t w1 = *reinterpret_cast<const uint32_t*>(v0 + T::BYTES + voff[j % T::R] + off);
        a[0] = fp8x2_to_bf16x2<false>(w0);
        a[1] = fp8x2_to_bf16x2<true>(w0);
        a[2] = fp8x2_to_bf16x2<false>(w1);
        a[3] = fp8x2_to_bf16x2<true>(w1);
      } else {
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(v0 + voff[j % T::R] + off);
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(v0 + T::BYTES + voff[j % T::R] + off);
        a = u32x4{a0[0], a0[1], a1[0], a1[1]};
      }
      return a;
    };
    // The products with V run at raised wave priority: a wavefront that
    // has reached them issues its MFMAs ahead of the others' softmax
    // arithmetic, which keeps the matrix unit fed.
    // Operand j + 1 is read while the products of operand j run; the
    // scheduling barrier keeps the compiler from hoisting all the reads
    // ahead of the products, which measured 8-10 % slower on the kernel.
    __builtin_amdgcn_s_setprio(1);
    u32x4 a = v_op(0);
#pragma unroll
    for (int j = 0; j < T::DC; ++j) {
      const u32x4 an = j + 1 < T::DC ? v_op(j + 1) : a;
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(bh), acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(bl), acc[j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      a = an;
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // A wavefront none of whose columns holds a member only brings its share
  // of each stage and meets the barriers.
  const bool busy = __builtin_amdgcn_readfirstlane(wave * MPW) < nmem;

  if (nst > 0) {
    // Stages 0 .. kStages - 2 in flight; stage s lands in buffer s %
    // kStages.  At the top of stage i this wavefront waits for its own two
    // loads of stage i, and the barrier then stands for everyone's; every
    // wavefront is also past stage i - 1, so its buffer takes stage
    // i + kStages - 1.  The loads and barriers run for whole groups of
    // kStages stages (past the last stage they move a valid tile nobody
    // reads), so that every path keeps the same loads in flight.
#pragma unroll
    for (int j = 0; j < kStages - 1; ++j) issue(j < nst ? j : nst - 1, j);
    for (int i0 = 0; i0 < nst; i0 += kStages) {
#pragma unroll
      for (int j = 0; j < kStages; ++j) {
        const int i = i0 + j;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (kStages - 2)));
        // A barrier without a memory fence: a fence would wait for every
        // load in flight, the later stages' included.  The memory clobber
        // keeps the compiler from moving LDS reads across it, and this
        // stage's data is covered by the wait above.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int nx = i + kStages - 1;
        issue(nx < nst ? nx : nst - 1, (j + kStages - 1) % kStages);
        if (busy) {
          const uint8_t* buf = stage_buf(j);
#pragma unroll
          for (int pp = 0; pp < T::TS / 2; ++pp) {
            const int t0 = i * T::TS + 2 * pp;
            if (t0 < ntiles) pair(buf, pp, t0 + 1 < ntiles);
          }
        }
      }
    }
    // No load may still be writing LDS when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }

  float ltot = l + __shfl_xor(l, 16, 64);
  ltot += __shfl_xor(ltot, 32, 64);
  if (bad) ltot = __builtin_nanf("");
  if (col_ok) {
    // O^T block j = R e + s holds on row 4 qd + i the dim
    // 16 (R e + ((4 qd / H) ^ s)) + H s + 4 qd % H + i.
    float* rec = p.partials + ((int64_t)(slot0 + mk) * p.num_q_heads + qh) * (D + 4);
#pragma unroll
    for (int j = 0; j < T::DC; ++j) {
      const int e = j / T::R, s_ = j % T::R;
      const int d0 = 16 * (T::R * e + (((4 * qd) / T::H) ^ s_)) + T::H * s_ + (4 * qd) % T::H;
      *reinterpret_cast<f32x4*>(rec + d0) = acc[j];
    }
    if (qd == 0) *reinterpret_cast<f32x4*>(rec + D) = f32x4{m, ltot, 0.f, 0.f};
  }
}

// One thread per (sequence, query head, 4 dims).
// One thread per (sequence, query head, 4 dims).  The parts are merged with
// a running maximum, kCombineBatch at a time: the slots of a batch are
// loaded together, then all of their records' (m, l) and acc pieces, so a
// sequence with up to kCombineBatch shared parts costs three dependent
// memory round trips (its part range, the slots, the records).
constexpr int kCombineBatch = 4;
__global__ __launch_bounds__(256) void combine_kernel(const CombineParams p) {
  const int q4 = p.head_dim / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)p.num_seqs * p.num_q_heads * q4) return;
  const int64_t row = gid / q4;                     // s * Hq + i
  const int d4 = (int)(gid - row * q4);
  const int s = (int)(row / p.num_q_heads), i = (int)(row - (int64_t)s * p.num_q_heads);
  const int D = p.head_dim;
  const int k0 = p.parts_off[s], k1 = p.parts_off[s + 1];
  const float lse_p = p.part_lse[row];
  const f32x4 out_p = reinterpret_cast<const f32x4*>(p.part_out + row * D)[d4];
  // The private part: normalized output out_p, weight 2^lse_p.
  float M = lse_p, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  if (lse_p != kNegInf) {
    num = out_p;
    den = 1.f;
  }
  bool bad = lse_p != lse_p;
  for (int kb = k0; kb < k1 && !bad; kb += kCombineBatch) {
    int slot[kCombineBatch];
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) slot[b] = p.parts[kb + b < k1 ? kb + b : kb];
    f32x4 acc[kCombineBatch];
    float m[kCombineBatch], l[kCombineBatch];
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      const bool ok = (unsigned)slot[b] < (unsigned)p.num_slots;
      if (kb + b < k1 && !ok) bad = true;
      const float* rec = p.partials + ((int64_t)(ok ? slot[b] : 0) * p.num_q_heads + i) * (D + 4);
      m[b] = rec[D];
      l[b] = rec[D + 1];
      acc[b] = reinterpret_cast<const f32x4*>(rec)[d4];
    }
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      if (kb + b < k1) {
        const float lse_k = m[b] + __builtin_amdgcn_logf(l[b]);
        const float m_new = __builtin_fmaxf(M, lse_k);
        const float a = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M - m_new);
        const float w = (lse_k == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(lse_k - m_new);
        num = num * a + acc[b] * (w * p.out_scale / l[b]);
        den = den * a + w;
        M = m_new;
      }
    }
  }
  f32x4 o;
  if (M == kNegInf) o = f32x4{0.f, 0.f, 0.f, 0.f};   // nothing to attend to
  else o = num * (1.f / den);
  if (bad) {
    const float nan = __builtin_nanf("");
    o = f32x4{nan, nan, nan, nan};                   // invalid length or slot: NaN rows
  }
  reinterpret_cast<f32x4*>(p.out + row * D)[d4] = o;
}

}  // namespace

hipError_t launch_segments(const SegmentParams& p, bool fp8, hipStream_t stream) {
  if (p.num_items == 0) return hipSuccess;
  const dim3 grid((unsigned)p.num_items), block(kSegThreads);
  if (p.head_dim == 128) {
    if (fp8) hipLaunchKernelGGL((segment_kernel<128, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((segment_kernel<128, false>), grid, block, 0, stream, p);
  } else {
    if (fp8) hipLaunchKernelGGL((segment_kernel<64, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((segment_kernel<64, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.num_seqs * p.num_q_heads * (p.head_dim / 4);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
