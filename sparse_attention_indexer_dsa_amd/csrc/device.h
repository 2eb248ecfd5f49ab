// device.h -- gfx950 device helpers shared by the indexer kernels: vector types
// for the MFMA operands, the order-preserving fp32 key, wave ballots/ranks, and
// the wave-level radix selection that keeps a candidate buffer's top K.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsaidx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { kBF16 = 1, kFP8 = 2 };

// fp32 -> uint32 such that a > b (as reals, -0 == +0 after canonicalisation)
// iff key(a) > key(b).  Key 0 is below every finite score, so it serves as the
// "accept everything" threshold.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }
// number of set bits of m in lanes below this one
__device__ __forceinline__ int rank_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
__device__ __forceinline__ int first_lane(uint64_t m) { return __ffsll((long long)m) - 1; }
__device__ __forceinline__ int shfl(int v, int src) { return __shfl(v, src, 64); }
__device__ __forceinline__ uint32_t shfl_u(uint32_t v, int src) {
  return (uint32_t)__shfl((int)v, src, 64);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (l >= o) v += t;
  }
  return v;
}

// Make this wave's earlier global stores visible to its later loads from other
// lanes (same CU: a workgroup-scope fence drains the store counter).
__device__ __forceinline__ void wave_mem_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// One radix digit step of the selection: given the entries whose key matches
// `prefix` on `pmask`, histogram digit (key >> shift) & (NBINS-1) into `hist`
// (NBINS counters in LDS owned by this wave) and find the digit holding the
// krem-th largest matching entry.  Updates prefix/pmask/krem; wave-uniform.
template <int NBINS>
__device__ __forceinline__ void radix_step(const uint32_t* keys, int n, uint32_t* hist, int shift,
                                           uint32_t& prefix, uint32_t& pmask, int& krem) {
  constexpr int PER = NBINS / 64;
  const int l = lane_id();
  uint32_t* mine = hist + l * PER;
#pragma unroll
  for (int b = 0; b < PER; b += 4) *(u32x4*)(mine + b) = u32x4{0u, 0u, 0u, 0u};
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint32_t dmask = NBINS - 1;
  int e = l;
  for (; e + 192 < n; e += 256) {
    uint32_t k0 = keys[e], k1 = keys[e + 64], k2 = keys[e + 128], k3 = keys[e + 192];
    if ((k0 & pmask) == prefix) atomicAdd(hist + ((k0 >> shift) & dmask), 1u);
    if ((k1 & pmask) == prefix) atomicAdd(hist + ((k1 >> shift) & dmask), 1u);
    if ((k2 & pmask) == prefix) atomicAdd(hist + ((k2 >> shift) & dmask), 1u);
    if ((k3 & pmask) == prefix) atomicAdd(hist + ((k3 >> shift) & dmask), 1u);
  }
  for (; e < n; e += 64) {
    uint32_t k0 = keys[e];
    if ((k0 & pmask) == prefix) atomicAdd(hist + ((k0 >> shift) & dmask), 1u);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint32_t c[PER];
  int local = 0;
#pragma unroll
  for (int b = 0; b < PER; b += 4) {
    u32x4 v = *(const u32x4*)(mine + b);
    c[b] = v[0]; c[b + 1] = v[1]; c[b + 2] = v[2]; c[b + 3] = v[3];
    local += (int)(v[0] + v[1] + v[2] + v[3]);
  }
  // entries in higher lanes' (higher) bins
  const int incl = wave_incl_scan(local);
  const int total = shfl(incl, 63);
  const int above = total - incl;
  const uint64_t hit = ballot(above < krem && above + local >= krem);
  const int L = first_lane(hit);
  int digit = 0, newk = 0;
  if (l == L) {
    int acc = above;
#pragma unroll
    for (int b = PER - 1; b >= 0; --b) {
      int cb = (int)c[b];
      if (acc + cb >= krem && newk == 0) { digit = l * PER + b; newk = krem - acc; }
      acc += cb;
    }
  }
  digit = shfl(digit, L);
  krem = shfl(newk, L);
  prefix |= (uint32_t)digit << shift;
  pmask |= dmask << shift;
}

// Keep the top K (by key descending, then by buffer position, i.e. ascending
// key index) of the n > K entries of a wave's candidate buffer, compacting them
// in place in their original order.  Returns the K-th largest key.
// `hist` holds 2048 LDS counters for this wave.  All 64 lanes must call it.
__device__ __forceinline__ uint32_t wave_select_topk(uint32_t* keys, int32_t* idx, int n, int K,
                                                     uint32_t* hist) {
  wave_mem_fence();
  uint32_t prefix = 0, pmask = 0;
  int krem = K;
  radix_step<2048>(keys, n, hist, 21, prefix, pmask, krem);
  radix_step<2048>(keys, n, hist, 10, prefix, pmask, krem);
  radix_step<1024>(keys, n, hist, 0, prefix, pmask, krem);
  const uint32_t kth = prefix;
  const int keep_eq = krem;  // entries equal to kth to keep, earliest first
  const int l = lane_id();
  int out = 0, eq_seen = 0;
  for (int base = 0; base < n; base += 64) {
    const int e = base + l;
    const bool in = e < n;
    uint32_t key = in ? keys[e] : 0u;
    int32_t id = in ? idx[e] : 0;
    const bool gt = in && key > kth;
    const bool eq = in && key == kth;
    const uint64_t eqm = ballot(eq);
    const bool keep = gt || (eq && eq_seen + rank_below(eqm) < keep_eq);
    eq_seen += popc(eqm);
    const uint64_t km = ballot(keep);
    if (keep) {
      const int p = out + rank_below(km);
      keys[p] = key;
      idx[p] = id;
    }
    out += popc(km);
  }
  wave_mem_fence();
  return kth;
}

}  // namespace dsaidx
