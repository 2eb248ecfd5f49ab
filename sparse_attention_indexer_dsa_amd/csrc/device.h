// device.h -- gfx950 device helpers shared by the indexer kernels: vector types
// for the MFMA operands, the order-preserving fp32 key, wave ballots/ranks, and
// the wave-level radix selection that keeps a candidate buffer's top K.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsaidx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer resource on gfx9 (32-bit data format, no swizzle):
// loads past num_records return zeros and stores past it are dropped.
constexpr int kBufferWord3 = 0x00020000;

enum { kBF16 = 1, kFP8 = 2 };

// fp32 -> uint32 such that a > b iff key(a) > key(b), for finite a, b other
// than -0: key(-0) is one below key(+0), so every kernel turns a -0 score
// into +0 (by adding +0) before it takes its key.  Key 0 is below every finite
// score, so it serves as the "accept everything" threshold.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ReLU on the fp32 bit pattern: negative floats are negative as int32 (and
// -0 is INT_MIN), so one v_max_i32 gives max(x, +0) for every finite x.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// sum_r w[r] * ReLU(acc[r]) over the 16 accumulators of one 32x32 MFMA tile,
// added to two interleaved partial sums.
__device__ __forceinline__ void gated_relu_sum16(const float* w, const v16f& acc, float& s0,
                                                 float& s1) {
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    s0 = fmaf(w[r], relu_bits(acc[r]), s0);
    s1 = fmaf(w[r + 1], relu_bits(acc[r + 1]), s1);
  }
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
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

// LDS words of one wave's selection histogram: 2048 16-bit counters, two per
// word (every candidate buffer holds fewer than 65536 entries).
constexpr int kSelectHistWords = 1024;

// Order LDS accesses of the lanes of one wave (a histogram's updates before
// its reads).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Zero the first NBINS/2 words of a wave's histogram (every lane its share).
template <int NBINS>
__device__ __forceinline__ void hist_zero(uint32_t* hist) {
  constexpr int PERW = NBINS / 2 / 64;
  uint32_t* mine = hist + lane_id() * PERW;
#pragma unroll
  for (int b = 0; b < PERW; b += 4) *(u32x4*)(mine + b) = u32x4{0u, 0u, 0u, 0u};
}

// One 16-bit histogram count (two per word) of order key k's digit
// (k >> shift) & (NBINS - 1).
template <int NBINS>
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t k, int shift) {
  const uint32_t bin = (k >> shift) & (NBINS - 1);
  atomicAdd(hist + (bin >> 1), 1u << ((bin & 1u) * 16u));
}

// Pick step of a radix digit: given a histogram of the digit (key >> shift)
// & (NBINS-1) over the entries that match `prefix` on `pmask`, find the digit
// holding the krem-th largest of them.  Updates prefix/pmask/krem and returns
// the number of entries with the chosen digit; wave-uniform.
template <int NBINS>
__device__ __forceinline__ int radix_pick(const uint32_t* hist, int shift, uint32_t& prefix,
                                          uint32_t& pmask, int& krem) {
  constexpr int PERW = NBINS / 2 / 64;  // words per lane
  constexpr int PER = 2 * PERW;         // bins per lane
  const int l = lane_id();
  const uint32_t* mine = hist + l * PERW;
  uint32_t c[PER];
  int local = 0;
#pragma unroll
  for (int b = 0; b < PERW; b += 4) {
    u32x4 v = *(const u32x4*)(mine + b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[2 * (b + q)] = v[q] & 0xFFFFu;
      c[2 * (b + q) + 1] = v[q] >> 16;
      local += (int)((v[q] & 0xFFFFu) + (v[q] >> 16));
    }
  }
  // entries in higher lanes' (higher) bins
  const int incl = wave_incl_scan(local);
  const int total = shfl(incl, 63);
  const int above = total - incl;
  const uint64_t hit = ballot(above < krem && above + local >= krem);
  const int L = first_lane(hit);
  int digit = 0, newk = 0, cnt = 0;
  if (l == L) {
    int acc = above;
#pragma unroll
    for (int b = PER - 1; b >= 0; --b) {
      int cb = (int)c[b];
      if (acc + cb >= krem && newk == 0) { digit = l * PER + b; newk = krem - acc; cnt = cb; }
      acc += cb;
    }
  }
  digit = shfl(digit, L);
  krem = shfl(newk, L);
  prefix |= (uint32_t)digit << shift;
  pmask |= (uint32_t)(NBINS - 1) << shift;
  return shfl(cnt, L);
}

// Count step of a radix digit over a candidate buffer of raw fp32 scores
// (compared through order_key): histogram digit (key >> shift) & (NBINS-1) of
// the entries whose key matches `prefix` on `pmask` into `hist` (this wave's
// kSelectHistWords LDS words, NBINS <= 2048 16-bit counters).
// B loads per lane are kept in flight (the buffer usually sits in HBM).
template <int NBINS, int B = 16>
__device__ __forceinline__ void radix_count(const uint32_t* keys, int n, uint32_t* hist, int shift,
                                            uint32_t prefix, uint32_t pmask) {
  const int l = lane_id();
  hist_zero<NBINS>(hist);
  wave_lds_sync();
  auto count = [&](uint32_t raw) {
    const uint32_t k = order_key(__uint_as_float(raw));
    if ((k & pmask) == prefix) {
      hist_add<NBINS>(hist, k, shift);
    }
  };
  // every batch, the last one too, issues all its loads before the first
  // use: a buffer costs ceil(n / (64 B)) memory round trips
  for (int e0 = l; e0 < n; e0 += B * 64) {
    uint32_t k[B];
#pragma unroll
    for (int u = 0; u < B; ++u) k[u] = e0 + 64 * u < n ? keys[e0 + 64 * u] : 0u;
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (e0 + 64 * u < n) count(k[u]);
  }
  wave_lds_sync();
}
// One radix digit step: count, then find the digit holding the krem-th
// largest matching entry.  Updates prefix/pmask/krem; wave-uniform.
template <int NBINS, int B = 16>
__device__ __forceinline__ void radix_step(const uint32_t* keys, int n, uint32_t* hist, int shift,
                                           uint32_t& prefix, uint32_t& pmask, int& krem) {
  radix_count<NBINS, B>(keys, n, hist, shift, prefix, pmask);
  radix_pick<NBINS>(hist, shift, prefix, pmask, krem);
}

// Keep the top K (by score descending, then by buffer position, i.e. ascending
// key index) of the n > K entries of a wave's candidate buffer (raw fp32 score
// bits + key indices), compacting them in place in their original order; n
// becomes the number kept.  Returns a threshold: no score at or below it can
// still enter the top K.
//   * slack >= 0 (a compaction during the stream): when the 22-bit key bucket
//     that holds the K-th best has at most K + slack entries at or above it,
//     the third digit is skipped and that whole bucket is kept; the threshold
//     is then the bucket's lowest value instead of the K-th best score.
//     slack < 0: exactly K are kept and the threshold is the K-th best score.
// `hist` is this wave's kSelectHistWords LDS words.  All 64 lanes must call it.
__device__ __forceinline__ float wave_keep_topk(uint32_t* keys, int32_t* idx, int& n, int K,
                                                uint32_t* hist, int slack) {
  wave_mem_fence();
  uint32_t prefix = 0, pmask = 0;
  int krem = K;
  radix_step<2048>(keys, n, hist, 21, prefix, pmask, krem);
  radix_count<2048>(keys, n, hist, 10, prefix, pmask);
  const int in_bucket = radix_pick<2048>(hist, 10, prefix, pmask, krem);
  // entries at or above the bucket: K - krem above it, in_bucket inside
  bool bucket = slack >= 0 && K - krem + in_bucket <= K + slack;
  if (bucket) {
    const float lo = key_to_float(prefix);
    bucket = lo == lo;  // a bucket whose lowest key is no number keeps the exact path
  }
  if (!bucket) radix_step<1024>(keys, n, hist, 0, prefix, pmask, krem);
  const uint32_t kth = prefix;  // exact: the K-th best key; bucket: its lowest key
  const int keep_eq = krem;     // exact: entries equal to kth to keep, earliest first
  const int l = lane_id();
  int out = 0, eq_seen = 0;
  constexpr int kU = 8;  // chunks of 64 loaded together
  for (int base = 0; base < n; base += 64 * kU) {
    uint32_t raw[kU];
    int32_t id[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = base + 64 * u + l;
      raw[u] = e < n ? keys[e] : 0u;
      id[u] = e < n ? idx[e] : 0;
    }
    // every load of the batch lands before the first store below overwrites
    // an earlier position of the same buffer
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = base + 64 * u + l;
      const bool in = e < n;
      const uint32_t key = order_key(__uint_as_float(raw[u]));
      const bool gt = in && key > kth;
      const bool eq = in && key == kth;
      const uint64_t eqm = ballot(eq);
      const bool keep = gt || (eq && (bucket || eq_seen + rank_below(eqm) < keep_eq));
      eq_seen += popc(eqm);
      const uint64_t km = ballot(keep);
      if (keep) {
        const int p = out + rank_below(km);
        keys[p] = raw[u];
        idx[p] = id[u];
      }
      out += popc(km);
    }
  }
  n = out;
  wave_mem_fence();
  return key_to_float(kth);
}

// A compaction during the stream may keep up to this many entries beyond K
// (the whole 22-bit key bucket of the K-th best) instead of a third pass; the
// buffers' headroom (cap - 192 >= 2K + 1856 entries before a compaction is
// due) leaves room for them.
constexpr int kCompactSlack = 256;

// The exact selection: keep the top K of n > K entries; returns the K-th
// largest score.
__device__ __forceinline__ float wave_select_topk(uint32_t* keys, int32_t* idx, int n, int K,
                                                  uint32_t* hist) {
  return wave_keep_topk(keys, idx, n, K, hist, -1);
}

// The output pass of a final selection: the entries of keys[0, n) above kth,
// and the first keep_eq equal to it (all of them when !select), written to
// oidx / osc in buffer order with index map(load_id(e)), then -1 / -inf
// padding up to K.  Loads are batched kU chunks of 64 per lane: load_id(e)
// is called for every in-range slot of a batch, then map on each result, so
// the loads of either stage are all in flight together.
template <int kU, typename LoadId, typename Map>
__device__ __forceinline__ void emit_kept(const uint32_t* keys, int n, int K, bool select, uint32_t kth,
                                          int keep_eq, int32_t* oidx, float* osc, LoadId load_id, Map map) {
  const int l = lane_id();
  int out = 0, eq_seen = 0;
  for (int base = 0; base < n; base += 64 * kU) {
    uint32_t raw[kU];
    int32_t id[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = base + 64 * u + l;
      raw[u] = e < n ? keys[e] : 0u;
      id[u] = e < n ? load_id(e) : 0;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = base + 64 * u + l;
      id[u] = e < n ? map(id[u]) : 0;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = base + 64 * u + l;
      const bool in = e < n;
      const uint32_t key = order_key(__uint_as_float(raw[u]));
      const bool eq = in && key == kth;
      const uint64_t eqm = ballot(eq);
      const bool keep = in && (!select || key > kth || (eq && eq_seen + rank_below(eqm) < keep_eq));
      eq_seen += popc(eqm);
      const uint64_t km = ballot(keep);
      if (keep) {
        const int p = out + rank_below(km);
        oidx[p] = id[u];
        if (osc) osc[p] = __uint_as_float(raw[u]);
      }
      out += popc(km);
    }
  }
  for (int p = out + l; p < K; p += 64) {
    oidx[p] = -1;
    if (osc) osc[p] = -__builtin_inff();
  }
}

// The final selection, written straight into a query's output row: the top
// K of the wave's n buffer entries (all of them when n <= K) in buffer order,
// i.e. ascending key index, then -1 / -inf padding up to K.  The buffer is
// read B entries per lane at a time (the caller's registers are free by now).
// osc may be null.  `hist` is this wave's kSelectHistWords LDS words.
template <int B>
__device__ __forceinline__ void wave_emit_topk(const uint32_t* keys, const int32_t* idx, int n,
                                               int K, uint32_t* hist, int32_t* oidx, float* osc) {
  wave_mem_fence();
  const bool select = n > K;
  uint32_t kth = 0;
  int keep_eq = 0;
  if (select) {
    uint32_t prefix = 0, pmask = 0;
    int krem = K;
    radix_step<2048, B>(keys, n, hist, 21, prefix, pmask, krem);
    radix_count<2048, B>(keys, n, hist, 10, prefix, pmask);
    const int in_bucket = radix_pick<2048>(hist, 10, prefix, pmask, krem);
    if (in_bucket == krem && prefix != 0u) {
      // the K-th best's 22-bit key bucket is taken whole: the top K are the
      // entries at or above its lowest key, and the last digit needs no pass
      kth = prefix - 1u;
      keep_eq = 0;
    } else {
      radix_step<1024, B>(keys, n, hist, 0, prefix, pmask, krem);
      kth = prefix;
      keep_eq = krem;
    }
  }
  emit_kept<B / 2>(keys, n, K, select, kth, keep_eq, oidx, osc, [&](int e) { return idx[e]; },
                   [](int32_t i) { return i; });
}

// The final selection over a wave's full score row: raw fp32 scores
// keys[0, n) (n < 65536) of candidates 0 .. n-1, whose top 11 order-key bits
// `hist` (this wave's kSelectHistWords LDS words, 2048 16-bit counters)
// already counts, so the first digit needs no pass over the row.  One pass
// then keeps the entries at or above the first digit's bin (every entry of
// the top K, and the rest of that bin) in place, in candidate order, with
// their indices pos(candidate) in ids[], and counts the second digit of the
// bin's entries; the third digit and the output pass run over that list
// only.  pos is called for every candidate of a batch together with the
// score loads, so a lookup it makes adds no round trip.  Writes the top K in
// candidate order, then the padding; osc may be null.
template <int B, typename Pos>
__device__ __forceinline__ void wave_emit_row(uint32_t* keys, int32_t* ids, int n, int K, uint32_t* hist,
                                              int32_t* oidx, float* osc, Pos pos) {
  wave_mem_fence();
  wave_lds_sync();
  if (n <= K) {
    emit_kept<B>(keys, n, K, false, 0u, 0, oidx, osc, pos, [](int32_t i) { return i; });
    return;
  }
  uint32_t prefix = 0, pmask = 0;
  int krem = K;
  radix_pick<2048>(hist, 21, prefix, pmask, krem);
  const uint32_t lo = prefix;  // lowest order key of the first digit's bin
  hist_zero<2048>(hist);
  wave_lds_sync();
  const int l = lane_id();
  int m = 0;
  for (int e0 = 0; e0 < n; e0 += B * 64) {
    uint32_t raw[B];
    int32_t id[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int e = e0 + 64 * u + l;
      raw[u] = e < n ? keys[e] : 0u;
      id[u] = e < n ? pos(e) : 0;
    }
    // slot m + rank <= e: an entry moves only down, onto a chunk this batch
    // has already read (or an earlier one)
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int e = e0 + 64 * u + l;
      const uint32_t k = order_key(__uint_as_float(raw[u]));
      const bool keep = e < n && k >= lo;
      if (keep && (k & pmask) == prefix) hist_add<2048>(hist, k, 10);
      const uint64_t km = ballot(keep);
      if (keep) {
        const int p = m + rank_below(km);
        keys[p] = raw[u];
        ids[p] = id[u];
      }
      m += popc(km);
    }
  }
  wave_mem_fence();
  wave_lds_sync();
  const int in_bucket = radix_pick<2048>(hist, 10, prefix, pmask, krem);
  if (in_bucket == krem && prefix != 0u) {
    // the K-th best's 22-bit bucket is taken whole (no last-digit pass)
    emit_kept<B>(keys, m, K, true, prefix - 1u, 0, oidx, osc, [&](int e) { return ids[e]; },
                 [](int32_t i) { return i; });
    return;
  }
  radix_step<1024, B>(keys, m, hist, 0, prefix, pmask, krem);
  emit_kept<B>(keys, m, K, true, prefix, krem, oidx, osc, [&](int e) { return ids[e]; },
               [](int32_t i) { return i; });
}

}  // namespace dsaidx
