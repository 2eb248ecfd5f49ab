// decode.hip -- decode-time indexer for gfx950: one new bf16 query per
// sequence scores its whole E4M3 key cache (ADIndex (Qi et al.), Section 3:
// O(L) work per decoding query), then the top-K of each row (Eq. (2)).
//
// decode_scan: the cache stream is the cost.  Each wavefront takes 32 keys at
// a time; lane l loads its key's k-half (d/2 bytes) straight into registers
// (two 32-key tiles in flight while two others are scored), widens E4M3 to
// bf16 exactly (every E4M3 value is a bf16 value) with
// v_cvt_scalef32_pk_bf16_fp8, and runs the bf16 MFMA with the query's heads on
// M.  ReLU, the gate-weighted head sum and the per-key scale follow in
// registers; the fp32 score row goes to the workspace and every score also
// counts into a per-row histogram of the top 12 bits of its order-preserving
// key (LDS, flushed to the row's global histogram once per workgroup).
//
// decode_select: one workgroup per row.  The row histogram gives the bin b*
// that holds the K-th best score and the count above it.  One pass over the
// row marks every score above b* in an LDS bitmap of the row and gathers the
// scores inside b* into LDS; two radix rounds over those candidates find the
// exact K-th score (ties: lower index first), and a prefix popcount of the
// bitmap writes the selected indices in ascending order.  Rows whose b* bin
// is too crowded for LDS take an exact multi-pass path over the row instead.
#include "device.h"
#include "launch.h"

namespace dsaidx {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecTilesPerWave = 8;  // a multiple of 4: tiles go in pairs
constexpr int kDecKeysPerBlock = kDecWaves * kDecTilesPerWave * 32;

template <int D>
struct DecTile {
  static constexpr int kVec = D / 2 / 16;  // 16-byte loads per lane per tile
  u32x4 v[kVec];
};

template <int MT, int D>
__global__ void __launch_bounds__(kDecThreads, 2) decode_scan_kernel(const DecodeArgs args) {
  constexpr int kSteps = D / 16;  // bf16 k-steps
  constexpr int kHalf = D / 2;    // fp8 bytes of a lane's k-half
  constexpr int kVec = DecTile<D>::kVec;
  __shared__ uint32_t s_hist[kDecHistBins];
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = tid & 63;
  const int h = l >> 5, col = l & 31;
  int64_t n = args.seq_lens[b];
  n = n < 0 ? 0 : (n > args.Nmax ? args.Nmax : n);
  const int64_t blk0 = (int64_t)blockIdx.x * kDecKeysPerBlock;
  if (blk0 >= n) return;
  for (int i = tid; i < kDecHistBins; i += kDecThreads) s_hist[i] = 0;

  v8bf a[MT][kSteps];
  float wv[MT][16];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int head = 32 * m + col;
    const bool hv = head < args.H;
    const uint8_t* qrow =
        (const uint8_t*)args.q + ((int64_t)b * args.H + (hv ? head : 0)) * (2 * D);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      u32x4 v = hv ? *(const u32x4*)(qrow + h * D + 16 * s) : u32x4{0, 0, 0, 0};
      a[m][s] = __builtin_bit_cast(v8bf, v);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hr = 32 * m + 8 * (r >> 2) + 4 * h + (r & 3);
      wv[m][r] = hr < args.H ? args.w[(int64_t)b * args.H + hr] : 0.0f;
    }
  }
  __syncthreads();

  const uint8_t* kbase = args.kc + (int64_t)b * args.Nmax * D;
  const float* sbase = args.k_scale + (int64_t)b * args.Nmax;
  float* lrow = args.logits + (int64_t)b * args.ld;

  // tile i of this wave covers keys blk0 + (i*kDecWaves + wave)*32 + [0, 32)
  auto key_of = [&](int i) __attribute__((always_inline)) { return blk0 + ((int64_t)i * kDecWaves + wave) * 32 + col; };
  auto load = [&](DecTile<D>& t, float& ks, int i) __attribute__((always_inline)) {
    const int64_t key = key_of(i);
    const bool kv = key < n;
#pragma unroll
    for (int v = 0; v < kVec; ++v)
      t.v[v] = kv ? *(const u32x4*)(kbase + key * D + h * kHalf + 16 * v) : u32x4{0, 0, 0, 0};
    ks = kv ? sbase[key] : 0.0f;
  };
  auto score = [&](const DecTile<D>& t, float ks, int i) __attribute__((always_inline)) {
    const int64_t key = key_of(i);
    v16f acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = v16f{};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      // fp8 bytes 8s .. 8s+7 of this lane's k-half -> 8 bf16 (exact)
      const uint32_t w0 = t.v[s >> 1][(s & 1) * 2], w1 = t.v[s >> 1][(s & 1) * 2 + 1];
      v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
      v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
      v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
      v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
      v8bf bf = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
      for (int m = 0; m < MT; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m][s], bf, acc[m], 0, 0, 0);
    }
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m) gated_relu_sum16(wv[m], acc[m], s0, s1);
    float sc = s0 + s1;
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc), false,
                                               false);
    sc = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * ks;
    sc += 0.0f;  // -0 -> +0
    if (l < 32 && key < n) {
      lrow[key] = sc;
      atomicAdd(&s_hist[order_key(sc) >> (32 - kDecHistBits)], 1u);
    }
  };

  // tiles in pairs: the next pair's loads are in flight while a pair is scored
  DecTile<D> ta0, ta1, tb0, tb1;
  float ka0, ka1, kb0, kb1;
  load(ta0, ka0, 0);
  load(ta1, ka1, 1);
#pragma unroll
  for (int i = 0; i < kDecTilesPerWave; i += 4) {
    load(tb0, kb0, i + 2);
    load(tb1, kb1, i + 3);
    score(ta0, ka0, i);
    score(ta1, ka1, i + 1);
    if (i + 4 < kDecTilesPerWave) {
      load(ta0, ka0, i + 4);
      load(ta1, ka1, i + 5);
    }
    score(tb0, kb0, i + 2);
    score(tb1, kb1, i + 3);
  }
  __syncthreads();
  uint32_t* ghist = args.hist + (int64_t)b * kDecHistBins;
  for (int i = tid; i < kDecHistBins; i += kDecThreads) {
    const uint32_t c = s_hist[i];
    if (c) atomicAdd(ghist + i, c);
  }
}

// ------------------------------------------------------------------ select

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kCandCap = 8192;       // LDS candidates of the threshold bin
constexpr int kBitmapWords = 16384;  // rows up to 524288 keys use the bitmap path

// Exclusive prefix sum over the workgroup (all threads call); `total` gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int& total) {
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int incl = wave_incl_scan(v);
  if (l == 63) s_tmp[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int t = s_tmp[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

// Per-thread runs of `per` consecutive bins (higher thread = higher bins):
// find the bin holding the krem-th largest entry.  s_res[0] = bin,
// s_res[1] = rank within the bin, s_res[2] = count of the bin.  All threads call.
template <typename F>
__device__ __forceinline__ void block_find_digit(int per, F bins, int krem, int* s_tmp,
                                                 int* s_res) {
  const int tid = threadIdx.x;
  int local = 0;
  for (int i = 0; i < per; ++i) local += bins(tid, i);
  int total;
  const int excl = block_excl_scan(local, s_tmp, total);
  const int above = total - excl - local;
  if (above < krem && above + local >= krem) {
    int acc = above;
    for (int i = per - 1; i >= 0; --i) {
      const int c = bins(tid, i);
      if (acc + c >= krem) {
        s_res[0] = tid * per + i;
        s_res[1] = krem - acc;
        s_res[2] = c;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

// One radix round over n LDS keys (only those matching prefix on pmask):
// digit (key >> shift) & (nbins-1).  Updates prefix/pmask/krem and returns the
// count of the chosen digit.
__device__ __forceinline__ int block_radix_lds(const uint32_t* keys, int n, int shift, int nbins,
                                               uint32_t& prefix, uint32_t& pmask, int& krem,
                                               uint32_t* s_h, int* s_tmp, int* s_res) {
  const int tid = threadIdx.x;
  const uint32_t dmask = (uint32_t)nbins - 1;
  for (int i = tid; i < nbins; i += kSelThreads) s_h[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kSelThreads) {
    const uint32_t k = keys[i];
    if ((k & pmask) == prefix) atomicAdd(&s_h[(k >> shift) & dmask], 1u);
  }
  __syncthreads();
  const int per = (nbins + kSelThreads - 1) / kSelThreads;
  block_find_digit(per, [&](int t, int i) { return t * per + i < nbins ? (int)s_h[t * per + i] : 0; },
                   krem, s_tmp, s_res);
  const int digit = s_res[0];
  krem = s_res[1];
  const int cnt = s_res[2];
  __syncthreads();
  prefix |= (uint32_t)digit << shift;
  pmask |= dmask << shift;
  return cnt;
}

// Exact multi-pass selection straight over the row in global memory (rows
// whose threshold bin does not fit in LDS, or longer than the bitmap).
__device__ void select_row_exact(const float* row, int64_t n, int K, int32_t* oidx, float* osc,
                                 uint32_t* s_h, int* s_tmp, int* s_res) {
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  uint32_t prefix = 0, pmask = 0;
  int krem = K;
  for (int round = 0; round < 3; ++round) {
    const int shift = round == 0 ? 21 : (round == 1 ? 10 : 0);
    const int nbins = round == 2 ? 1024 : 2048;
    const uint32_t dmask = (uint32_t)nbins - 1;
    for (int i = tid; i < nbins; i += kSelThreads) s_h[i] = 0;
    __syncthreads();
    for (int64_t e = tid; e < n; e += kSelThreads) {
      const uint32_t key = order_key(row[e]);
      if ((key & pmask) == prefix) atomicAdd(&s_h[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    const int per = nbins / kSelThreads;
    block_find_digit(per, [&](int t, int i) { return (int)s_h[t * per + i]; }, krem, s_tmp, s_res);
    prefix |= (uint32_t)s_res[0] << shift;
    pmask |= dmask << shift;
    krem = s_res[1];
    __syncthreads();
  }
  const uint32_t kth = prefix;
  const int keep_eq = krem;
  // ordered emission: each wave owns a contiguous segment of the row
  const int64_t seg = ((n + kSelWaves - 1) / kSelWaves + 63) / 64 * 64;
  const int64_t s0 = (int64_t)wave * seg, s1 = s0 + seg < n ? s0 + seg : n;
  int gt = 0, eq = 0;
  for (int64_t base = s0; base < s1; base += 64) {
    const int64_t e = base + l;
    const bool in = e < s1;
    const uint32_t key = in ? order_key(row[e]) : 0u;
    gt += popc(ballot(in && key > kth));
    eq += popc(ballot(in && key == kth));
  }
  if (l == 0) {
    s_res[4 + wave] = gt;
    s_res[4 + kSelWaves + wave] = eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
  for (int w2 = 0; w2 < wave; ++w2) {
    gt_before += s_res[4 + w2];
    eq_before += s_res[4 + kSelWaves + w2];
  }
  int out = gt_before + (eq_before < keep_eq ? eq_before : keep_eq);
  int eq_seen = eq_before;
  for (int64_t base = s0; base < s1; base += 64) {
    const int64_t e = base + l;
    const bool in = e < s1;
    const float v = in ? row[e] : 0.0f;
    const uint32_t key = order_key(v);
    const bool g = in && key > kth;
    const bool q = in && key == kth;
    const uint64_t qm = ballot(q);
    const bool keep = g || (q && eq_seen + rank_below(qm) < keep_eq);
    eq_seen += popc(qm);
    const uint64_t km = ballot(keep);
    const int p = out + rank_below(km);
    if (keep && p < K) {
      oidx[p] = (int32_t)e;
      if (osc) osc[p] = v;
    }
    out += popc(km);
  }
}

// One row: top-K of logits[0..n) by (score desc, index asc), indices ascending.
__global__ void __launch_bounds__(kSelThreads) decode_select_kernel(const DecodeArgs args) {
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ uint32_t s_ckey[kCandCap];
  __shared__ int32_t s_cidx[kCandCap];
  __shared__ uint32_t s_h[2048];
  __shared__ int s_tmp[kSelWaves];
  __shared__ int s_res[4 + 2 * kSelWaves];
  __shared__ int s_count;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, l = tid & 63;
  int64_t n = args.seq_lens[b];
  n = n < 0 ? 0 : (n > args.Nmax ? args.Nmax : n);
  const int K = args.K;
  const float* row = args.logits + (int64_t)b * args.ld;
  int32_t* oidx = args.out_idx + (int64_t)b * K;
  float* osc = args.out_score ? args.out_score + (int64_t)b * K : nullptr;
  if (n <= K) {
    for (int p = tid; p < K; p += kSelThreads) {
      oidx[p] = p < n ? p : -1;
      if (osc) osc[p] = p < n ? row[p] : -__builtin_inff();
    }
    return;
  }

  // 1. threshold bin b* from the row histogram (4 bins per thread)
  const uint32_t* ghist = args.hist + (int64_t)b * kDecHistBins;
  constexpr int kPer = kDecHistBins / kSelThreads;
  block_find_digit(kPer, [&](int t, int i) { return (int)ghist[t * kPer + i]; }, K, s_tmp, s_res);
  const uint32_t bstar = (uint32_t)s_res[0];
  const int need = s_res[1];   // entries of bin b* that are selected
  const int inbin = s_res[2];  // entries in bin b*
  constexpr int kShift = 32 - kDecHistBits;
  __syncthreads();
  if (inbin > kCandCap || n > 32 * (int64_t)kBitmapWords) {
    select_row_exact(row, n, K, oidx, osc, s_h, s_tmp, s_res);
    return;
  }

  // 2. one pass: bitmap bits for everything above b*, LDS candidates inside b*
  const int words = (int)((n + 31) / 32);
  for (int i = tid; i < words; i += kSelThreads) s_bits[i] = 0;
  if (tid == 0) s_count = 0;
  __syncthreads();
  for (int64_t wbase = (int64_t)(tid - l) * 4; wbase < n; wbase += (int64_t)kSelThreads * 4) {
    const int64_t e0 = wbase + l * 4;  // whole waves iterate together (ballots below)
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (e0 + 3 < n) {
      const float4 f = *(const float4*)(row + e0);
      v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
      for (int u = 0; u < 4; ++u) v[u] = e0 + u < n ? row[e0 + u] : 0.0f;
    }
    uint32_t mine = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = e0 + u < n;
      const uint32_t key = order_key(v[u]);
      const uint32_t bin = key >> kShift;
      if (in && bin > bstar) mine |= 1u << ((e0 + u) & 31);
      const bool cand = in && bin == bstar;
      const uint64_t m = ballot(cand);
      if (m) {
        const int fl = first_lane(m);
        int base = 0;
        if (l == fl) base = atomicAdd(&s_count, popc(m));
        base = shfl(base, fl);
        if (cand) {
          const int p = base + rank_below(m);
          if (p < kCandCap) {
            s_ckey[p] = key;
            s_cidx[p] = (int32_t)(e0 + u);
          }
        }
      }
    }
    if (mine && e0 < n) atomicOr(&s_bits[e0 >> 5], mine);
  }
  __syncthreads();
  const int nc = s_count < kCandCap ? s_count : kCandCap;

  // 3. exact K-th key among the candidates (the low 20 bits, two rounds)
  uint32_t prefix = bstar << kShift, pmask = ~0u << kShift;
  int krem = need;
  block_radix_lds(s_ckey, nc, 10, 1024, prefix, pmask, krem, s_h, s_tmp, s_res);
  const int n_eq = block_radix_lds(s_ckey, nc, 0, 1024, prefix, pmask, krem, s_h, s_tmp, s_res);
  const uint32_t kth = prefix;
  const int keep_eq = krem;  // of the n_eq candidates equal to kth keep the keep_eq lowest indices

  // 4. ties at kth: the keep_eq-th largest ~index among them is the cut
  uint32_t idx_cut = 0u;  // an equal key is kept when ~index >= idx_cut
  if (keep_eq < n_eq) {
    uint32_t tp = 0, tm = 0;
    int tk = keep_eq;
    for (int round = 0; round < 3; ++round) {
      const int shift = round == 0 ? 21 : (round == 1 ? 10 : 0);
      const int nbins = round == 2 ? 1024 : 2048;
      const uint32_t dmask = (uint32_t)nbins - 1;
      for (int i = tid; i < nbins; i += kSelThreads) s_h[i] = 0;
      __syncthreads();
      for (int i = tid; i < nc; i += kSelThreads) {
        if (s_ckey[i] != kth) continue;
        const uint32_t r = ~(uint32_t)s_cidx[i];
        if ((r & tm) == tp) atomicAdd(&s_h[(r >> shift) & dmask], 1u);
      }
      __syncthreads();
      const int per = (nbins + kSelThreads - 1) / kSelThreads;
      block_find_digit(per,
                       [&](int t, int i) { return t * per + i < nbins ? (int)s_h[t * per + i] : 0; },
                       tk, s_tmp, s_res);
      tp |= (uint32_t)s_res[0] << shift;
      tm |= dmask << shift;
      tk = s_res[1];
      __syncthreads();
    }
    idx_cut = tp;
  }
  for (int i = tid; i < nc; i += kSelThreads) {
    const uint32_t key = s_ckey[i];
    const uint32_t e = (uint32_t)s_cidx[i];
    if (key > kth || (key == kth && ~e >= idx_cut)) atomicOr(&s_bits[e >> 5], 1u << (e & 31));
  }
  __syncthreads();

  // 5. emit in ascending index: prefix popcount over the bitmap
  const int wpt = (words + kSelThreads - 1) / kSelThreads;
  const int w0 = tid * wpt, w1 = w0 + wpt < words ? w0 + wpt : words;
  int cnt = 0;
  for (int wd = w0; wd < w1; ++wd) cnt += __popc(s_bits[wd]);
  int total;
  int pos = block_excl_scan(cnt, s_tmp, total);
  for (int wd = w0; wd < w1; ++wd) {
    uint32_t bits = s_bits[wd];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      const int64_t e = (int64_t)wd * 32 + bit;
      if (pos < K) {
        oidx[pos] = (int32_t)e;
        if (osc) osc[pos] = row[e];
      }
      ++pos;
    }
  }
}

template <int MT, int D>
static hipError_t launch_dec(const DecodeArgs& a, hipStream_t stream) {
  const int64_t bx = (a.Nmax + kDecKeysPerBlock - 1) / kDecKeysPerBlock;
  if (a.B <= 0) return hipSuccess;
  hipError_t e = launch_fill_i32((int32_t*)a.hist, (int64_t)a.B * kDecHistBins, 0, stream);
  if (e != hipSuccess) return e;
  if (bx > 0)
    hipLaunchKernelGGL((decode_scan_kernel<MT, D>), dim3((unsigned)bx, (unsigned)a.B),
                       dim3(kDecThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_select_kernel, dim3((unsigned)a.B), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int MT = a.H <= 32 ? 1 : 2;
  if (MT == 1) {
    if (a.d == 64) return launch_dec<1, 64>(a, stream);
    return launch_dec<1, 128>(a, stream);
  }
  if (a.d == 64) return launch_dec<2, 64>(a, stream);
  return launch_dec<2, 128>(a, stream);
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

}  // namespace dsaidx
