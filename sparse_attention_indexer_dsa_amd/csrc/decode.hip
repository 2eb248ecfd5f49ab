// decode.hip -- decode-time indexer for gfx950: one new bf16 query per
// sequence scores its whole E4M3 key cache (ADIndex (Qi et al.), Section 3:
// O(L) work per decoding query), then the top-K of each row (Eq. (2)).
//
// decode_scan: the cache stream is the cost.  Each wavefront takes 32 keys at
// a time; lane l loads its key's k-half (d/2 bytes) straight into registers,
// widens E4M3 to bf16 exactly (every E4M3 value is a bf16 value) with
// v_cvt_scalef32_pk_bf16_fp8, and runs the bf16 MFMA with the query's heads on
// M.  ReLU, the gate-weighted head sum and the per-key scale follow in
// registers; the fp32 score row goes to a workspace row of the caller.
// decode_select: one workgroup per row, three radix-digit rounds (11/11/10
// bits of the order-preserving key) over an LDS histogram find the K-th score;
// two ordered passes emit the selected indices in ascending order.
#include "device.h"
#include "launch.h"

namespace dsaidx {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecTilesPerWave = 8;
constexpr int kDecKeysPerBlock = kDecWaves * kDecTilesPerWave * 32;

template <int MT, int D>
__global__ void __launch_bounds__(kDecThreads, 2) decode_scan_kernel(const DecodeArgs args) {
  constexpr int kSteps = D / 16;  // bf16 k-steps
  constexpr int kHalf = D / 2;    // fp8 bytes of a lane's k-half
  constexpr int kVec = kHalf / 16;
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int l = threadIdx.x & 63;
  const int h = l >> 5, col = l & 31;
  int64_t n = args.seq_lens[b];
  n = n < 0 ? 0 : (n > args.Nmax ? args.Nmax : n);
  const int64_t blk0 = (int64_t)blockIdx.x * kDecKeysPerBlock;
  if (blk0 >= n) return;

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

  const uint8_t* kbase = args.kc + (int64_t)b * args.Nmax * D;
  const float* sbase = args.k_scale + (int64_t)b * args.Nmax;
  float* lrow = args.logits + (int64_t)b * args.ld;

  for (int i = 0; i < kDecTilesPerWave; ++i) {
    const int64_t key = blk0 + ((int64_t)i * kDecWaves + wave) * 32 + col;
    if (blk0 + ((int64_t)i * kDecWaves + wave) * 32 >= n) break;
    const bool kv = key < n;
    u32x4 raw[kVec];
#pragma unroll
    for (int v = 0; v < kVec; ++v)
      raw[v] = kv ? *(const u32x4*)(kbase + key * D + h * kHalf + 16 * v) : u32x4{0, 0, 0, 0};
    const float ks = kv ? sbase[key] : 0.0f;
    v16f acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = v16f{};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      // fp8 bytes 8s .. 8s+7 of this lane's k-half -> 8 bf16 (exact)
      const uint32_t w0 = raw[s >> 1][(s & 1) * 2], w1 = raw[s >> 1][(s & 1) * 2 + 1];
      v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
      v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
      v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
      v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
      v8bf bf = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
      for (int m = 0; m < MT; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m][s], bf, acc[m], 0, 0, 0);
    }
    float sc = 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc = fmaf(wv[m][r], fmaxf(acc[m][r], 0.0f), sc);
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc), false,
                                               false);
    sc = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * ks;
    sc += 0.0f;  // -0 -> +0
    if (l < 32 && kv) lrow[key] = sc;
  }
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// One row: top-K of logits[0..n) by (score desc, index asc), indices ascending.
__global__ void __launch_bounds__(kSelThreads) decode_select_kernel(const DecodeArgs args) {
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[2048];
  __shared__ int s_digit, s_krem;
  __shared__ int s_gt[kSelWaves], s_eq[kSelWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
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

  uint32_t prefix = 0, pmask = 0;
  int krem = K;
  for (int round = 0; round < 3; ++round) {
    const int shift = round == 0 ? 21 : (round == 1 ? 10 : 0);
    const int nbins = round == 2 ? 1024 : 2048;
    const uint32_t dmask = (uint32_t)nbins - 1;
    for (int i = tid; i < 2048; i += kSelThreads) s_hist[i] = 0;
    __syncthreads();
    for (int64_t e = (int64_t)tid * 4; e < n; e += (int64_t)kSelThreads * 4) {
      float v[4];
      if (e + 3 < n) {
        float4 f = *(const float4*)(row + e);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
      } else {
        for (int u = 0; u < 4; ++u) v[u] = e + u < n ? row[e + u] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t key = order_key(v[u]);
        if (e + u < n && (key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int per = nbins / 64;
      int local = 0;
      for (int i = 0; i < per; ++i) local += (int)s_hist[l * per + i];
      const int incl = wave_incl_scan(local);
      const int above = shfl(incl, 63) - incl;
      const uint64_t hit = ballot(above < krem && above + local >= krem);
      const int L = first_lane(hit);
      if (l == L) {
        int acc = above;
        for (int i = per - 1; i >= 0; --i) {
          const int c = (int)s_hist[l * per + i];
          if (acc + c >= krem) { s_digit = l * per + i; s_krem = krem - acc; break; }
          acc += c;
        }
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_digit << shift;
    pmask |= dmask << shift;
    krem = s_krem;
    __syncthreads();
  }
  const uint32_t kth = prefix;
  const int keep_eq = krem;

  // ordered emission: each wave owns a contiguous segment
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
  if (l == 0) { s_gt[wave] = gt; s_eq[wave] = eq; }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
  for (int w2 = 0; w2 < wave; ++w2) { gt_before += s_gt[w2]; eq_before += s_eq[w2]; }
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

template <int MT, int D>
static hipError_t launch_dec(const DecodeArgs& a, hipStream_t stream) {
  const int64_t bx = (a.Nmax + kDecKeysPerBlock - 1) / kDecKeysPerBlock;
  if (a.B <= 0) return hipSuccess;
  if (bx > 0)
    hipLaunchKernelGGL((decode_scan_kernel<MT, D>), dim3((unsigned)bx, (unsigned)a.B),
                       dim3(kDecThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
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
