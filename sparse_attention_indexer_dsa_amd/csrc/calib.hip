// calib.hip -- statistics for the layer-wise reuse calibration of ADIndex (Qi
// et al.), Section 4.1 Eq. (4): the union size of the reference top-K index
// sets of each group of G consecutive queries, and (Appendix B.4) the overlap
// of two index sets per query, the coverage of a reuse result.
//
// Index sets are the indexer's output rows: ascending token indices, then -1.
// union: one workgroup per group marks its G*K indices in an LDS bitmap
// (2^18 tokens per pass, more passes only for longer sequences) and counts
// the set bits.  overlap: one workgroup per row stages the second set in LDS;
// each thread binary-searches the first entry of its run of the first set and
// walks the rest.
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
  __shared__ int s_hi;
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int32_t* rows = idx + g * G * (int64_t)K;
  const int n = G * K;  // a multiple of 4
  constexpr int kU = 4;  // 16-byte loads per thread in flight
  int count = 0;
  // one pass per 2^18 tokens; the first pass also finds the group's largest
  // index, so sequences of up to 2^18 tokens read the group once
  for (int base = 0;; base += kBitmapTokens) {
    for (int w = tid; w < kBitmapWords; w += kCalThreads) s_bits[w] = 0u;
    if (tid == 0) s_hi = -1;
    __syncthreads();
    int hi = -1;
    for (int e0 = 4 * tid; e0 < n; e0 += 4 * kCalThreads * kU) {
      int4 q[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int e = e0 + 4 * kCalThreads * u;
        q[u] = e < n ? *reinterpret_cast<const int4*>(rows + e) : make_int4(-1, -1, -1, -1);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int v[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          hi = max(hi, v[c]);
          const int d = v[c] - base;
          if (v[c] >= 0 && d >= 0 && d < kBitmapTokens) atomicOr(&s_bits[d >> 5], 1u << (d & 31));
        }
      }
    }
    atomicMax(&s_hi, hi);
    __syncthreads();
    for (int w = tid; w < kBitmapWords; w += kCalThreads) count += __popc(s_bits[w]);
    const bool done = s_hi < base + kBitmapTokens;
    __syncthreads();  // s_bits and s_hi are rewritten by the next pass
    if (done) break;
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
  // b into LDS (4-byte loads, a thread's all in flight together), and this
  // thread's run of a (8 consecutive entries when K = 8 * threads; K % 4 == 0,
  // a 16-byte aligned) loaded alongside
  int nb = 0;
#pragma unroll 8
  for (int e = tid; e < K; e += kCalThreads) {
    const int32_t v = br[e];
    s_b[e] = v;
    nb += v >= 0;
  }
  const int run = ((K + kCalThreads - 1) / kCalThreads + 3) / 4 * 4;  // entries of a per thread
  const int a0 = tid * run, a1 = min(a0 + run, K);
  constexpr int kPre = 2;  // 16-byte pieces of the run loaded before the barrier
  int4 pre[kPre];
#pragma unroll
  for (int p = 0; p < kPre; ++p)
    pre[p] = a0 + 4 * p < a1 ? *reinterpret_cast<const int4*>(ar + a0 + 4 * p) : make_int4(-1, -1, -1, -1);
  nb = block_sum(nb, s_tmp);  // also orders the LDS writes before the reads
  // each thread merges its run of a (ascending) with b: one binary search for
  // the run's first entry, then a linear walk
  int hits = 0;
  if (a0 < a1 && pre[0].x >= 0) {
    int lo = 0, hi = nb;  // valid entries of b are s_b[0, nb), ascending
    const int32_t first = pre[0].x;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_b[mid] < first) lo = mid + 1;
      else hi = mid;
    }
    auto walk = [&](const int4& q) __attribute__((always_inline)) {
      const int32_t v[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (v[u] < 0) break;
        while (lo < nb && s_b[lo] < v[u]) ++lo;
        hits += lo < nb && s_b[lo] == v[u];
      }
    };
#pragma unroll
    for (int p = 0; p < kPre; ++p) walk(pre[p]);
    for (int e = a0 + 4 * kPre; e < a1; e += 4) walk(*reinterpret_cast<const int4*>(ar + e));
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
