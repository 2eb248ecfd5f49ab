// calib.hip -- statistics for the layer-wise reuse calibration of ADIndex (Qi
// et al.), Section 4.1 Eq. (4): the union size of the reference top-K index
// sets of each group of G consecutive queries, and (Appendix B.4) the overlap
// of two index sets per query, the coverage of a reuse result.
//
// Index sets are the indexer's output rows: ascending token indices, then -1.
// union: one workgroup per group marks its G*K indices in an LDS bitmap
// (2^18 tokens per pass, more passes for longer sequences) and counts the
// set bits.  overlap: one workgroup per row stages the second set in LDS and
// binary-searches every entry of the first.
#include "device.h"
#include "launch.h"

namespace dsaidx {

namespace {

constexpr int kCalThreads = 256;
constexpr int kBitmapWords = 8192;  // 2^18 token bits, 32 KB
constexpr int kBitmapTokens = kBitmapWords * 32;

// sum of v over the workgroup (all threads call; two barriers)
__device__ __forceinline__ int block_sum(int v, int* s_tmp) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int incl = wave_incl_scan(v);
  if (l == 63) s_tmp[wave] = incl;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kCalThreads / 64; ++w) t += s_tmp[w];
  __syncthreads();
  return t;
}

__global__ void __launch_bounds__(kCalThreads) union_kernel(const int32_t* idx, int K, int G,
                                                            int32_t* out) {
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ int s_tmp[kCalThreads / 64];
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int32_t* rows = idx + g * G * (int64_t)K;
  const int n = G * K;
  int hi = -1;  // the largest index of the group: passes needed
  for (int e = 4 * tid; e < n; e += 4 * kCalThreads) {
    const int4 q = *reinterpret_cast<const int4*>(rows + e);
    hi = max(max(hi, max(q.x, q.y)), max(q.z, q.w));
  }
  __shared__ int s_hi;
  if (tid == 0) s_hi = -1;
  __syncthreads();
  atomicMax(&s_hi, hi);
  __syncthreads();
  hi = s_hi;
  int count = 0;
  for (int base = 0; base <= hi; base += kBitmapTokens) {
    // only the words up to the group's largest index are touched
    const int words = min(kBitmapWords, (hi - base) / 32 + 1);
    for (int w = tid; w < words; w += kCalThreads) s_bits[w] = 0u;
    __syncthreads();
    for (int e = 4 * tid; e < n; e += 4 * kCalThreads) {  // K*G is a multiple of 4
      const int4 q = *reinterpret_cast<const int4*>(rows + e);
      const int v[4] = {q.x - base, q.y - base, q.z - base, q.w - base};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (v[u] >= 0 && v[u] < kBitmapTokens) atomicOr(&s_bits[v[u] >> 5], 1u << (v[u] & 31));
    }
    __syncthreads();
    for (int w = tid; w < words; w += kCalThreads) count += __popc(s_bits[w]);
    __syncthreads();
  }
  const int total = block_sum(count, s_tmp);
  if (tid == 0) out[g] = total;
}

__global__ void __launch_bounds__(kCalThreads) overlap_kernel(const int32_t* a, const int32_t* b, int K,
                                                              int32_t* out) {
  extern __shared__ int32_t s_b[];  // K entries
  __shared__ int s_tmp[kCalThreads / 64];
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const int32_t* ar = a + r * K;
  const int32_t* br = b + r * K;
  int nb = 0;
  for (int e = tid; e < K; e += kCalThreads) {
    const int32_t v = br[e];
    s_b[e] = v;
    nb += v >= 0;
  }
  nb = block_sum(nb, s_tmp);  // also orders the LDS writes before the reads
  // each thread merges a run of 4 consecutive entries of a (ascending) with
  // b: one binary search for the run's first entry, then a linear walk
  int hits = 0;
  for (int e = 4 * tid; e < K; e += 4 * kCalThreads) {
    const int4 q = *reinterpret_cast<const int4*>(ar + e);
    const int32_t v[4] = {q.x, q.y, q.z, q.w};
    if (v[0] < 0) continue;
    int lo = 0, hi = nb;  // valid entries of b are s_b[0, nb), ascending
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_b[mid] < v[0]) lo = mid + 1;
      else hi = mid;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (v[u] < 0) break;
      while (lo < nb && s_b[lo] < v[u]) ++lo;
      hits += lo < nb && s_b[lo] == v[u];
    }
  }
  const int total = block_sum(hits, s_tmp);
  if (tid == 0) out[r] = total;
}

}  // namespace

hipError_t launch_union_sizes(const int32_t* idx, int64_t groups, int K, int G, int32_t* out,
                              hipStream_t stream) {
  if (groups <= 0) return hipSuccess;
  hipLaunchKernelGGL(union_kernel, dim3((unsigned)groups), dim3(kCalThreads), 0, stream, idx, K, G, out);
  return hipGetLastError();
}

hipError_t launch_topk_overlap(const int32_t* a, const int32_t* b, int64_t n, int K, int32_t* out,
                               hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(overlap_kernel, dim3((unsigned)n), dim3(kCalThreads), (size_t)K * 4, stream, a, b, K, out);
  return hipGetLastError();
}

}  // namespace dsaidx
