// probe.hip -- the two streams the kernels are measured against:
//   * the plain read stream (memory-bound kernels): every byte of a buffer
//     read once with coalesced 16-byte loads, eight per lane in flight, and
//     nothing else (an XOR of the words so the loads cannot be dropped; one
//     word per workgroup is written);
//   * the matrix-core stream (the prefill kernels): back-to-back 32x32x64
//     E4M3 or 32x32x16 bf16 MFMAs on register operands into kMfmaChains independent
//     accumulators per wave, no memory traffic in the loop, with each wave's
//     shader-clock and 100 MHz constant-clock counts around its loop, so a run
//     gives the sustained rate and the clock the SIMDs ran at.  The operand
//     words' mask sets how much of the number range they span: the chip's
//     power limit makes the sustained rate depend on the data.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "dsa_indexer.h"
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

constexpr int kMfmaChains = 4;
constexpr int kMfmaPadWords = 24576;  // 96 KiB of LDS: one workgroup per CU

// Operand word i of the probe: a 32-bit mix of i, masked.
__device__ __forceinline__ uint32_t probe_word(uint32_t i, uint32_t mask) {
  uint32_t h = i * 0x9E3779B1u;
  h ^= h >> 15;
  h *= 0x85EBCA77u;
  h ^= h >> 13;
  return h & mask;
}

template <int kWavesPerSimd, int DT>
__global__ void __launch_bounds__(256 * kWavesPerSimd) mfma_probe_kernel(int iters, uint32_t mask, float* out,
                                                                           uint64_t* clocks) {
  __shared__ uint32_t s_pad[kMfmaPadWords];
  const int tid = threadIdx.x, l = tid & 63;
  // operands: E4M3 bytes or bf16 halves from a mixed index under the
  // caller's mask, varied per lane, written through LDS so the allocation
  // stays
  for (int i = tid; i < kMfmaPadWords; i += blockDim.x) s_pad[i] = probe_word((uint32_t)i, mask);
  __syncthreads();
  // E4M3: 32x32x64 on 8-word operands; bf16: 32x32x16 on 4-word operands
  constexpr int kW = DT == kFP8 ? 8 : 4;
  typedef int vw __attribute__((ext_vector_type(kW)));
  vw a[2], b[2];
#pragma unroll
  for (int k = 0; k < kW; ++k) {
    a[0][k] = (int)s_pad[l * 8 + k];
    a[1][k] = (int)s_pad[512 + l * 8 + k];
    b[0][k] = (int)s_pad[1024 + l * 8 + k];
    b[1][k] = (int)s_pad[1536 + l * 8 + k];
  }
  v16f acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = v16f{};
  __syncthreads();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) {
      if constexpr (DT == kFP8)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[c & 1], b[(c >> 1) & 1], acc[c], 0, 0, 0, 0, 0, 0);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[c & 1]),
                                                         __builtin_bit_cast(v8bf, b[(c >> 1) & 1]), acc[c], 0, 0, 0);
    }
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += acc[c][i];
  out[(int64_t)blockIdx.x * blockDim.x + tid] = sum;
  if (l == 0) {
    const int64_t wv = (int64_t)blockIdx.x * (blockDim.x / 64) + (tid >> 6);
    clocks[2 * wv] = c1 - c0;
    clocks[2 * wv + 1] = r1 - r0;
  }
}

template <int DT>
hipError_t launch_mfma_probe_dt(int iters, int waves_per_simd, int nblocks, uint32_t mask, float* out,
                                uint64_t* clocks, hipStream_t stream) {
  const dim3 grid((unsigned)nblocks), block((unsigned)(256 * waves_per_simd));
  switch (waves_per_simd) {
    case 1: hipLaunchKernelGGL((mfma_probe_kernel<1, DT>), grid, block, 0, stream, iters, mask, out, clocks); break;
    case 2: hipLaunchKernelGGL((mfma_probe_kernel<2, DT>), grid, block, 0, stream, iters, mask, out, clocks); break;
    default: hipLaunchKernelGGL((mfma_probe_kernel<4, DT>), grid, block, 0, stream, iters, mask, out, clocks); break;
  }
  return hipGetLastError();
}

}  // namespace

static_assert(kFP8 == DSAIDX_FP8_E4M3 && kBF16 == DSAIDX_BF16, "the probe takes the ABI's dtype codes");

hipError_t launch_mfma_probe(int dtype, int iters, int waves_per_simd, int nblocks, uint32_t mask, float* out,
                             uint64_t* clocks, hipStream_t stream) {
  return dtype == kFP8 ? launch_mfma_probe_dt<kFP8>(iters, waves_per_simd, nblocks, mask, out, clocks, stream)
                       : launch_mfma_probe_dt<kBF16>(iters, waves_per_simd, nblocks, mask, out, clocks, stream);
}

hipError_t launch_read_probe(const void* p, int64_t bytes, uint32_t* out, int nblocks, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int ntail = (int)(bytes - n16 * 16);
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)nblocks), dim3(kProbeThreads), 0, stream,
                     (const u32x4*)p, n16, (const uint8_t*)p + n16 * 16, ntail, out);
  return hipGetLastError();
}

}  // namespace dsaidx
