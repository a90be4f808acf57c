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
// chunk is loaded once into LDS (double-buffered) and used by all the
// workgroup's wavefronts; a wavefront
// holds MPW = 16 / G members' query groups as the 16 columns of its MFMA
// tiles (S^T = K Q^T with 16x16x32 bf16, O^T = V^T P^T with 16x16x16 bf16,
// P split into bf16 hi + lo), the same operand layouts as the paged decode
// kernel reads from registers, here read from LDS.  Each (member, chunk)
// gets a partial record {acc[D], m, l} per query head of h.
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

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ i16x4 as_i16x4(u32x2 v) { return __builtin_bit_cast(i16x4, v); }

template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// hi = p truncated to bf16, lo = (p - hi) truncated to bf16.
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

template <int D, bool FP8>
struct SegTile {
  static constexpr int EB = FP8 ? 1 : 2;
  static constexpr int BYTES = kSub * D * EB;        // one (block, head, sub-block) tile
  static constexpr int KLD = FP8 ? D / 64 : D / 32;  // 16-byte K operand loads per lane
  static constexpr int QK = D / 32;                  // 16x16x32 MFMAs per tile (K Q^T)
  static constexpr int DC = D / 16;                  // 16-row blocks of O^T
  static constexpr int R = FP8 ? 4 : 2;              // dim blocks per 16-byte V piece
  static constexpr int VLD = DC / R;
  static constexpr int PIECES = BYTES / 16;          // 16-byte pieces per tile (<= 256)
  static_assert(PIECES <= 64 * PA_CASCADE_WAVES, "one piece per thread");
};

constexpr int kSegThreads = 64 * PA_CASCADE_WAVES;

template <int D, bool FP8>
__global__ __launch_bounds__(kSegThreads) void segment_kernel(const SegmentParams p) {
  using T = SegTile<D, FP8>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2 * T::BYTES];
  const int32_t* it = p.items + (int64_t)blockIdx.x * 8;
  const int blk_off = it[0], nblk = it[1], mem_off = it[2], nmem = it[3], h = it[4], slot0 = it[5];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qd = lane >> 4, col = lane & 15;
  const int G = p.group, MPW = p.mpw;
  const int subs = p.block_size / kSub;
  const int ntiles = nblk * subs;
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
      const u32x4 v = *reinterpret_cast<const u32x4*>(qb + imm);
      qop[c] = as_bf16x8(col_ok ? v : u32x4{0u, 0u, 0u, 0u});
    }
  }

  // A block id outside the pool reads tile 0 instead and marks the records
  // NaN, as the paged decode marks such rows.
  u32x4 kreg = {0u, 0u, 0u, 0u}, vreg = {0u, 0u, 0u, 0u};
  bool bad = false;
  auto gload = [&](int t) {
    const int b = t / subs, sub = t - b * subs;
    const int blk = p.seg_blocks[blk_off + b];
    const bool ok = (unsigned)blk < (unsigned)p.num_blocks;
    bad |= !ok;
    const int64_t tile = ok ? (int64_t)blk * p.blk_stride + (int64_t)(h * subs + sub) * T::BYTES : 0;
    if (tid < T::PIECES) {
      kreg = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.k_cache + tile) + tid);
      vreg = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.v_cache + tile) + tid);
    }
  };
  auto lstore = [&](int b) {
    if (tid < T::PIECES) {
      reinterpret_cast<u32x4*>(lds[b])[tid] = kreg;
      reinterpret_cast<u32x4*>(lds[b] + T::BYTES)[tid] = vreg;
    }
  };

  float m = kNegInf, l = 0.f;
  f32x4 acc[T::DC];
#pragma unroll
  for (int dc = 0; dc < T::DC; ++dc) acc[dc] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) gload(t + 1);
    const uint8_t* kt = lds[t & 1];
    const uint8_t* vt = lds[t & 1] + T::BYTES;
    // Logits, base 2: lane holds tokens 4 qd + i of the tile, column col.
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < T::KLD; ++c) {
      const u32x4 kw = *reinterpret_cast<const u32x4*>(kt + c * 1024 + lane * 16);
      if constexpr (FP8) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 w;
          w[0] = fp8x2_to_bf16x2<false>(kw[2 * half]);
          w[1] = fp8x2_to_bf16x2<true>(kw[2 * half]);
          w[2] = fp8x2_to_bf16x2<false>(kw[2 * half + 1]);
          w[3] = fp8x2_to_bf16x2<true>(kw[2 * half + 1]);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w), qop[2 * c + half], s, 0, 0, 0);
        }
      } else {
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kw), qop[c], s, 0, 0, 0);
      }
    }
    float z[4];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = s[i] * p.qk_scale;
      mx = __builtin_fmaxf(mx, z[i]);
    }
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (__builtin_amdgcn_ballot_w64(mx > m + kSlack) != 0) {
      const float m_new = __builtin_fmaxf(m, mx);
      const float alpha = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dc = 0; dc < T::DC; ++dc) acc[dc] *= alpha;
    }
    float pz[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pz[i] = __builtin_amdgcn_exp2f(z[i] - m);
    l += (pz[0] + pz[1]) + (pz[2] + pz[3]);
    u32x2 p_hi, p_lo;
    split_p(pz, p_hi, p_lo);
    // O^T += V^T P^T: lane (col, qd) reads tokens 4 qd .. 4 qd + 3 of dims
    // 16 (R e + r) + col, as the cache tile stores them.
#pragma unroll
    for (int e = 0; e < T::VLD; ++e) {
      const u32x4 vw = *reinterpret_cast<const u32x4*>(vt + e * 1024 + (col * 4 + qd) * 16);
#pragma unroll
      for (int r = 0; r < T::R; ++r) {
        u32x2 a;
        if constexpr (FP8) {
          a[0] = fp8x2_to_bf16x2<false>(vw[r]);
          a[1] = fp8x2_to_bf16x2<true>(vw[r]);
        } else {
          a[0] = vw[2 * r];
          a[1] = vw[2 * r + 1];
        }
        const int dc = e * T::R + r;
        acc[dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_i16x4(a), as_i16x4(p_hi), acc[dc], 0, 0, 0);
        acc[dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_i16x4(a), as_i16x4(p_lo), acc[dc], 0, 0, 0);
      }
    }
    if (t + 1 < ntiles) lstore((t + 1) & 1);
    __syncthreads();
  }

  float ltot = l + __shfl_xor(l, 16, 64);
  ltot += __shfl_xor(ltot, 32, 64);
  if (bad) ltot = __builtin_nanf("");
  if (col_ok) {
    float* rec = p.partials + ((int64_t)(slot0 + mk) * p.num_q_heads + qh) * (D + 4);
#pragma unroll
    for (int dc = 0; dc < T::DC; ++dc) *reinterpret_cast<f32x4*>(rec + 16 * dc + 4 * qd) = acc[dc];
    if (qd == 0) *reinterpret_cast<f32x4*>(rec + D) = f32x4{m, ltot, 0.f, 0.f};
  }
}

// One thread per (sequence, query head, 4 dims).
__global__ __launch_bounds__(256) void combine_kernel(const CombineParams p) {
  const int q4 = p.head_dim / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)p.num_seqs * p.num_q_heads * q4) return;
  const int64_t row = gid / q4;                     // s * Hq + i
  const int d4 = (int)(gid - row * q4);
  const int s = (int)(row / p.num_q_heads), i = (int)(row - (int64_t)s * p.num_q_heads);
  const int D = p.head_dim;
  const int k0 = p.parts_off[s], k1 = p.parts_off[s + 1];
  float lse_p = p.part_lse[row];
  float M = lse_p;
  for (int k = k0; k < k1; ++k) {
    if ((unsigned)p.parts[k] >= (unsigned)p.num_slots) {
      lse_p = __builtin_nanf("");
      break;
    }
    const float* rec = p.partials + ((int64_t)p.parts[k] * p.num_q_heads + i) * (D + 4);
    M = __builtin_fmaxf(M, rec[D] + __builtin_amdgcn_logf(rec[D + 1]));
  }
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (lse_p != kNegInf) {
    const float w = __builtin_amdgcn_exp2f(lse_p - M);
    num = reinterpret_cast<const f32x4*>(p.part_out + row * D)[d4] * w;
    den = w;
  }
  for (int k = k0; k < k1 && lse_p == lse_p; ++k) {
    const float* rec = p.partials + ((int64_t)p.parts[k] * p.num_q_heads + i) * (D + 4);
    const float lk = rec[D + 1];
    const float w = __builtin_amdgcn_exp2f(rec[D] + __builtin_amdgcn_logf(lk) - M);
    num += reinterpret_cast<const f32x4*>(rec)[d4] * (w * p.out_scale / lk);
    den += w;
  }
  f32x4 o;
  if (M == kNegInf) o = f32x4{0.f, 0.f, 0.f, 0.f};   // nothing to attend to
  else o = num * (1.f / den);
  if (lse_p != lse_p) o = f32x4{lse_p, lse_p, lse_p, lse_p};   // invalid length or slot: NaN rows
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
