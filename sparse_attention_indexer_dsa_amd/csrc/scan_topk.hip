// scan_topk.hip -- streaming lightning-indexer score + top-K for gfx950.
//
// One wavefront owns one query row and walks that query's candidate keys in
// ascending key index, 32 keys per step:
//   * MFMA with the query's heads on M and 32 keys on N (ADIndex (Qi et al.),
//     Section 3, Eq. (1): the per-head dot products q_{t,j} . k_s), bf16
//     v_mfma_f32_32x32x16_bf16 or fp8 v_mfma_f32_32x32x64_f8f6f4, fp32
//     accumulation; H <= 64 heads are zero-padded to 32 or 64 rows;
//   * ReLU and the gate-weighted head sum in registers: a lane holds 16 heads
//     of each 32-head tile for one key, the other half of the heads sits in
//     lane l^32 and one permlane32 swap completes the sum; per-token fp8
//     scales multiply after the sum (positive scales commute with ReLU);
//   * streaming top-K (Eq. (2)): a score enters the query's candidate buffer
//     only if it beats the running threshold (the K-th best so far); keys
//     arrive in ascending index, so a strict ">" keeps the lower index on ties.
//     When the buffer fills, a wave radix select keeps the best K in order.
// The 4 waves of a workgroup own 4 consecutive queries that share most of
// their candidates: the workgroup stages each 32-key tile once in LDS
// (double-buffered).  The T x T score matrix is never written anywhere.
//
// The same kernel serves three uses, picked by its arguments:
//   dense prefill     candidates 0..t of query t                    (Eq. (2))
//   group scan        queries = group anchors (q-bar, w-bar, Eq. (8)),
//                     top-P of the anchor prefix = the bank         (Eq. (13))
//   bank refinement   candidates = the group's bank, then t+1..i    (Eq. (14))
#include "device.h"
#include "launch.h"

namespace dsaidx {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWavesPerBlock * 64;
constexpr int kTileKeys = 32;
constexpr int kHistBins = 2048;

template <int DT, int MT, int D>
struct ScanCfg {
  static constexpr int kRowBytes = DT == kBF16 ? 2 * D : D;  // bytes of one key row
  static constexpr int kLdsRow = kRowBytes + 16;             // padded LDS row stride
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kChunks = kTileKeys * kChunksPerRow;  // 16-byte chunks per tile
  static constexpr int kLoads = (kChunks + kThreads - 1) / kThreads;
  static constexpr int kSteps = DT == kBF16 ? D / 16 : D / 64;  // MFMA k-steps over d
  static constexpr int kHalf = DT == kBF16 ? D : D / 2;         // bytes of a lane's k-half
};

template <int DT>
struct AFrag;
template <>
struct AFrag<kBF16> { typedef v8bf type; };
template <>
struct AFrag<kFP8> { typedef v8i type; };

template <int DT>
__device__ __forceinline__ v16f mfma(const typename AFrag<DT>::type& a,
                                     const typename AFrag<DT>::type& b, v16f c) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Candidate c of the workgroup -> key index.  Dense: c.  Bank: bank[c] for
// c < bank_len, then the post-anchor tokens anchor+1, anchor+2, ...
__device__ __forceinline__ int64_t cand_token(int64_t c, const int32_t* bank, int bank_len,
                                              int64_t anchor) {
  if (!bank) return c;
  return c < bank_len ? (int64_t)bank[c] : anchor + 1 + (c - bank_len);
}

template <int DT, int MT, int D>
__global__ void __launch_bounds__(kThreads, 2) scan_topk_kernel(const ScanArgs args) {
  using C = ScanCfg<DT, MT, D>;
  using Frag = typename AFrag<DT>::type;
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][kTileKeys * C::kLdsRow];
  __shared__ int32_t s_tok[2][kTileKeys];
  __shared__ float s_kscale[2][kTileKeys];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[kWavesPerBlock][kHistBins];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = tid & 63;
  const int h = l >> 5;   // which half of the k range / which 16 of each 32 heads
  const int col = l & 31;  // MFMA column = key within the tile

  // queries of this workgroup: the longest candidate lists are launched first
  const int64_t j_hi = args.nq - (int64_t)blockIdx.x * kWavesPerBlock - 1;  // highest row
  const int64_t j = j_hi - (kWavesPerBlock - 1) + wave;                      // this wave's row
  const bool active = j >= 0;
  const int64_t j_lo = j_hi - (kWavesPerBlock - 1) < 0 ? 0 : j_hi - (kWavesPerBlock - 1);

  // candidate list of the workgroup
  const int32_t* bank = nullptr;
  int bank_len = 0;
  int64_t anchor = 0;
  const int64_t t_hi = args.pos0 + j_hi * args.pos_stride;
  int64_t ncand_blk;
  if (args.bank) {
    const int64_t grp = j_lo / args.group;  // all 4 rows share one group
    anchor = args.pos0 + grp * args.group;
    bank = args.bank + grp * args.bank_stride;
    bank_len = (int)min((int64_t)args.bank_stride, anchor + 1);
    ncand_blk = bank_len + (t_hi - anchor);
  } else {
    ncand_blk = t_hi + 1;
  }
  const int64_t t_me = args.pos0 + (active ? j : j_lo) * args.pos_stride;
  const int64_t ncand_me = args.bank ? bank_len + (t_me - anchor) : t_me + 1;
  const int ntiles = (int)((ncand_blk + kTileKeys - 1) / kTileKeys);

  // ---- this wave's query: A fragments and gate weights in registers
  Frag a[MT][C::kSteps];
  float wv[MT][16];
  {
    float qs = 1.0f;
    if (DT == kFP8 && active) qs = args.q_scale[j];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int head = 32 * m + col;
      const bool hv = active && head < args.H;
      const uint8_t* qrow = (const uint8_t*)args.q +
                            ((active ? j : 0) * (int64_t)args.H + (hv ? head : 0)) * C::kRowBytes;
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) {
        if constexpr (DT == kBF16) {
          u32x4 v = hv ? *(const u32x4*)(qrow + h * C::kHalf + 16 * s) : u32x4{0, 0, 0, 0};
          a[m][s] = __builtin_bit_cast(v8bf, v);
        } else {
          u32x4 v0 = hv ? *(const u32x4*)(qrow + h * C::kHalf + 32 * s) : u32x4{0, 0, 0, 0};
          u32x4 v1 = hv ? *(const u32x4*)(qrow + h * C::kHalf + 32 * s + 16) : u32x4{0, 0, 0, 0};
          v8i t;
          t[0] = v0[0]; t[1] = v0[1]; t[2] = v0[2]; t[3] = v0[3];
          t[4] = v1[0]; t[5] = v1[1]; t[6] = v1[2]; t[7] = v1[3];
          a[m][s] = t;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int hr = 32 * m + 8 * (r >> 2) + 4 * h + (r & 3);
        wv[m][r] = (active && hr < args.H) ? args.w[j * (int64_t)args.H + hr] * qs : 0.0f;
      }
    }
  }

  uint32_t* ckey = args.cand_key + (active ? j : 0) * (int64_t)args.cap;
  int32_t* cidx = args.cand_idx + (active ? j : 0) * (int64_t)args.cap;
  uint32_t* hist = s_hist[wave];
  int cnt = 0;          // entries in the candidate buffer (wave-uniform)
  uint32_t thr = 0u;    // keys must exceed this to enter (wave-uniform)

  // ---- cooperative tile loader: global -> registers -> LDS
  u32x4 stage[C::kLoads];
  int32_t stage_tok = 0;
  float stage_ks = 1.0f;
  auto load_tile = [&](int it) {
    const int64_t base = (int64_t)it * kTileKeys;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int c = tid + i * kThreads;
      stage[i] = u32x4{0, 0, 0, 0};
      if (c < C::kChunks) {
        const int r = c / C::kChunksPerRow, p = c % C::kChunksPerRow;
        const int64_t cand = base + r;
        if (cand < ncand_blk) {
          const int64_t tok = cand_token(cand, bank, bank_len, anchor);
          stage[i] = *(const u32x4*)((const uint8_t*)args.k + tok * C::kRowBytes + p * 16);
        }
      }
    }
    if (tid < kTileKeys) {
      const int64_t cand = base + tid;
      stage_tok = cand < ncand_blk ? (int32_t)cand_token(cand, bank, bank_len, anchor) : INT32_MAX;
      stage_ks = (DT == kFP8 && cand < ncand_blk) ? args.k_scale[stage_tok] : 1.0f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int c = tid + i * kThreads;
      if (c < C::kChunks) {
        const int r = c / C::kChunksPerRow, p = c % C::kChunksPerRow;
        *(u32x4*)(&s_tile[buf][r * C::kLdsRow + p * 16]) = stage[i];
      }
    }
    if (tid < kTileKeys) {
      s_tok[buf][tid] = stage_tok;
      s_kscale[buf][tid] = stage_ks;
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntiles) load_tile(it + 1);

    const int64_t tbase = (int64_t)it * kTileKeys;
    if (active && tbase < ncand_me) {
      v16f acc[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = v16f{};
      const uint8_t* brow = &s_tile[buf][col * C::kLdsRow + h * C::kHalf];
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) {
        Frag b;
        if constexpr (DT == kBF16) {
          b = __builtin_bit_cast(v8bf, *(const u32x4*)(brow + 16 * s));
        } else {
          u32x4 v0 = *(const u32x4*)(brow + 32 * s);
          u32x4 v1 = *(const u32x4*)(brow + 32 * s + 16);
          b[0] = v0[0]; b[1] = v0[1]; b[2] = v0[2]; b[3] = v0[3];
          b[4] = v1[0]; b[5] = v1[1]; b[6] = v1[2]; b[7] = v1[3];
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = mfma<DT>(a[m][s], b, acc[m]);
      }
      // ReLU + gate-weighted head sum (Eq. (1)), this lane's 16*MT heads
      float sc = 0.0f;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc = fmaf(wv[m][r], fmaxf(acc[m][r], 0.0f), sc);
      // the other 16*MT heads of this key live in lane l ^ 32
      {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc), false,
                                                   false);
        sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      if constexpr (DT == kFP8) sc *= s_kscale[buf][col];
      sc += 0.0f;  // -0 -> +0
      const int32_t tok = s_tok[buf][col];
      const uint32_t key = order_key(sc);
      const bool take = (l < 32) && (tbase + col < ncand_me) && ((int64_t)tok <= t_me) && key > thr;
      const uint64_t tm = ballot(take);
      if (tm) {
        if (take) {
          const int p = cnt + rank_below(tm);
          ckey[p] = key;
          cidx[p] = tok;
        }
        cnt += popc(tm);
        if (cnt > args.cap - kTileKeys) {
          thr = wave_select_topk(ckey, cidx, cnt, args.K, hist);
          cnt = args.K;
        }
      }
    }

    if (it + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!active) return;
  if (cnt > args.K) {
    wave_select_topk(ckey, cidx, cnt, args.K, hist);
    cnt = args.K;
  } else {
    wave_mem_fence();
  }
  int32_t* oidx = args.out_idx + j * (int64_t)args.out_stride;
  float* osc = args.out_score ? args.out_score + j * (int64_t)args.out_stride : nullptr;
  for (int p = l; p < args.K; p += 64) {
    const bool v = p < cnt;
    oidx[p] = v ? cidx[p] : -1;
    if (osc) osc[p] = v ? key_to_float(ckey[p]) : -__builtin_inff();
  }
}

template <int DT, int MT, int D>
static hipError_t launch_t(const ScanArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.nq + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((scan_topk_kernel<DT, MT, D>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_scan_topk(const ScanArgs& a, int dtype, hipStream_t stream) {
  const int MT = a.H <= 32 ? 1 : 2;
  if (dtype == kBF16) {
    if (MT == 1) {
      if (a.d == 32) return launch_t<kBF16, 1, 32>(a, stream);
      if (a.d == 64) return launch_t<kBF16, 1, 64>(a, stream);
      return launch_t<kBF16, 1, 128>(a, stream);
    }
    if (a.d == 32) return launch_t<kBF16, 2, 32>(a, stream);
    if (a.d == 64) return launch_t<kBF16, 2, 64>(a, stream);
    return launch_t<kBF16, 2, 128>(a, stream);
  }
  if (MT == 1) {
    if (a.d == 64) return launch_t<kFP8, 1, 64>(a, stream);
    return launch_t<kFP8, 1, 128>(a, stream);
  }
  if (a.d == 64) return launch_t<kFP8, 2, 64>(a, stream);
  return launch_t<kFP8, 2, 128>(a, stream);
}

}  // namespace dsaidx
