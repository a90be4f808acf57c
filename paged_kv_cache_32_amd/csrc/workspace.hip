// Check of a decode workspace's merge counters.
//
// Every pa_decode call that runs to completion leaves the counters of its
// workspace at zero (the wavefront that merges a unit, or a group of its
// pieces, rearms the counter it used).  A non-zero counter therefore means
// the workspace was never zero-filled or a call on it did not complete, and
// later calls on it would merge too early.  This counts such words.
#include "../../include/pa.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kCheckThreads = 1024;

// One workgroup: each thread counts the non-zero words at a stride of the
// workgroup, then the counts are summed in LDS and stored by thread 0.
__global__ __launch_bounds__(kCheckThreads) void count_nonzero_kernel(const uint32_t* words, int64_t n,
                                                                      int32_t* out) {
  __shared__ int32_t part[kCheckThreads / 64];
  int32_t c = 0;
  for (int64_t i = threadIdx.x; i < n; i += kCheckThreads) c += words[i] != 0u ? 1 : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t t = 0;
    for (int k = 0; k < kCheckThreads / 64; ++k) t += part[k];
    *out = t;
  }
}

}  // namespace

}  // namespace pa

extern "C" pa_status pa_decode_workspace_check(const void* workspace, size_t workspace_bytes, int32_t num_seqs,
                                               int32_t num_kv_heads, int32_t* nonzero, void* stream) {
  if (!workspace || !nonzero) return PA_ERR_NULL;
  if (num_seqs < 0 || num_kv_heads <= 0) return PA_ERR_SHAPE;
  const size_t region = pa::counter_region_bytes((int64_t)num_seqs * num_kv_heads) +
                        (size_t)pa::kGroupCounters * sizeof(int32_t);
  if (workspace_bytes < region) return PA_ERR_WORKSPACE;
  hipLaunchKernelGGL(pa::count_nonzero_kernel, dim3(1), dim3(pa::kCheckThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint32_t*>(workspace), (int64_t)(region / sizeof(uint32_t)), nonzero);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
