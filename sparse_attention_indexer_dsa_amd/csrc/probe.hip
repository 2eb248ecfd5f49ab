// probe.hip -- the plain read stream that the memory-bound kernels are
// measured against: every byte of a buffer read once with coalesced 16-byte
// loads, eight per lane in flight, and nothing else (an XOR of the words so
// the loads cannot be dropped; one word per workgroup is written).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "launch.h"

namespace dsaidx {

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 8;

__global__ void __launch_bounds__(kProbeThreads) read_probe_kernel(const u32x4* p, int64_t n16,
                                                                   const uint8_t* tail, int ntail,
                                                                   uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = p[i];
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) x ^= tail[threadIdx.x];
  // the workgroup's XOR: lanes, then waves through LDS
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  __shared__ uint32_t s_x[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int wv = 0; wv < kProbeThreads / 64; ++wv) r ^= s_x[wv];
    out[blockIdx.x] = r;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* p, int64_t bytes, uint32_t* out, int nblocks, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int ntail = (int)(bytes - n16 * 16);
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)nblocks), dim3(kProbeThreads), 0, stream,
                     (const u32x4*)p, n16, (const uint8_t*)p + n16 * 16, ntail, out);
  return hipGetLastError();
}

}  // namespace dsaidx
