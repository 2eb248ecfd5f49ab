// group_pool.hip -- the training-free group query of ADIndex (Qi et al.),
// Section 5 ablation 2 and Appendix B.3-B.4: a frozen DSA indexer builds a
// group's token bank from the mean of the group's own indexer queries (head by
// head) and of their gate weights, in place of a trained group indexer.
//
// Memory-bound and tiny beside the scans it feeds: one workgroup row per group,
// each thread summing one 16-byte chunk (8 bf16) of the H*d query over the G
// member queries in fp64, which is exact for 16 bf16 values unless their
// magnitudes span more than 2^40 (and for the fp32 gates unless theirs span
// more than 2^25), then scaling by 1/G (exact, G a power of two).  The pooled
// query and gates are that mean rounded once to the nearest bf16 / fp32 (ties
// to even): the pooled query decides integer results (which keys enter the
// bank), so it is the correctly rounded mean, not one sum order's rounding.
#include "device.h"
#include "launch.h"

namespace dsaidx {

namespace {

constexpr int kPoolThreads = 256;

__device__ __forceinline__ double lo_bf16(uint32_t v) { return (double)__uint_as_float(v << 16); }
__device__ __forceinline__ double hi_bf16(uint32_t v) { return (double)__uint_as_float(v & 0xFFFF0000u); }

// The bf16 nearest to x (ties to the even significand), for |x| below the
// largest bf16: with x's binary exponent ex clamped to >= -126, the bf16 values
// there are the multiples of 2^(ex-7); x is scaled to that grid, rounded to an
// integer (v_rndne_f64: nearest, ties to even) and scaled back, all exact.
__device__ __forceinline__ uint16_t bf16_nearest_f64(double x) {
  if (x == 0.0) return (uint16_t)(__double_as_longlong(x) >> 48);  // +-0
  const int ex = max(__builtin_amdgcn_frexp_exp(x) - 1, -126);
  const double v = __builtin_ldexp(__builtin_rint(__builtin_ldexp(x, 7 - ex)), ex - 7);
  return (uint16_t)(__float_as_uint((float)v) >> 16);  // v has <= 8 significant bits
}

template <int G>
__global__ void __launch_bounds__(kPoolThreads) pool_mean_kernel(const PoolArgs a) {
  const int64_t grp = a.g0 + blockIdx.y;
  const int nchunk = a.H * a.d / 8;  // 16-byte chunks of one query row
  const int c = blockIdx.x * kPoolThreads + threadIdx.x;
  const double inv = 1.0 / (double)G;
  if (c < nchunk) {
    const uint4* src = reinterpret_cast<const uint4*>(a.q) + grp * G * nchunk + c;
    uint4 v[G];
#pragma unroll
    for (int i = 0; i < G; ++i) v[i] = src[(int64_t)i * nchunk];
    double s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = 0.0;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      s[0] += lo_bf16(v[i].x); s[1] += hi_bf16(v[i].x);
      s[2] += lo_bf16(v[i].y); s[3] += hi_bf16(v[i].y);
      s[4] += lo_bf16(v[i].z); s[5] += hi_bf16(v[i].z);
      s[6] += lo_bf16(v[i].w); s[7] += hi_bf16(v[i].w);
    }
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = (uint32_t)bf16_nearest_f64(s[2 * j] * inv) | ((uint32_t)bf16_nearest_f64(s[2 * j + 1] * inv) << 16);
    reinterpret_cast<uint4*>(a.qbar)[(int64_t)blockIdx.y * nchunk + c] =
        make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (blockIdx.x == 0 && threadIdx.x < a.H) {
    const float* src = a.w + grp * G * a.H + threadIdx.x;
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < G; ++i) s += (double)src[(int64_t)i * a.H];
    a.wbar[(int64_t)blockIdx.y * a.H + threadIdx.x] = (float)(s * inv);
  }
}

}  // namespace

hipError_t launch_pool_mean(const PoolArgs& args, hipStream_t stream) {
  if ((args.H * args.d) % 8 || args.H > kPoolThreads) return hipErrorInvalidValue;
  const int nchunk = args.H * args.d / 8;
  const int bx = (nchunk + kPoolThreads - 1) / kPoolThreads;
  constexpr int64_t kGroupsPerLaunch = 32768;  // grid y limit
  for (int64_t s = 0; s < args.ngroups; s += kGroupsPerLaunch) {
    PoolArgs a = args;
    a.g0 = args.g0 + s;
    a.ngroups = args.ngroups - s < kGroupsPerLaunch ? args.ngroups - s : kGroupsPerLaunch;
    a.qbar = (uint8_t*)args.qbar + s * args.H * args.d * 2;
    a.wbar = args.wbar + s * args.H;
    const dim3 grid((unsigned)bx, (unsigned)a.ngroups);
    switch (a.G) {
      case 4: hipLaunchKernelGGL(pool_mean_kernel<4>, grid, dim3(kPoolThreads), 0, stream, a); break;
      case 8: hipLaunchKernelGGL(pool_mean_kernel<8>, grid, dim3(kPoolThreads), 0, stream, a); break;
      case 16: hipLaunchKernelGGL(pool_mean_kernel<16>, grid, dim3(kPoolThreads), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dsaidx
