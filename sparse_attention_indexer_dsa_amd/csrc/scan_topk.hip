// scan_topk.hip -- streaming lightning-indexer score + top-K for gfx950.
//
// One wavefront owns one query row and walks that query's candidate keys in
// ascending key index:
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
// The WPB waves of a workgroup own WPB consecutive queries that share most of
// their candidates.  The workgroup streams 64-key tiles of K through a
// three-stage LDS ring fed from a three-deep register ring: a tile's global
// loads are issued four tiles before it is scored and land in LDS two tiles
// before, so HBM/MALL latency hides behind two tiles of MFMA work.  Inside a
// wave the MFMAs of the next 32-key sub-tile are interleaved with the ReLU and
// head sums of the current one, so the matrix cores and the VALU work at the
// same time.  The T x T score matrix is never written anywhere.
//
// The same kernel serves three uses, picked by its arguments:
//   dense prefill     candidates 0..t of query t                    (Eq. (2))
//   group scan        queries = group anchors (q-bar, w-bar, Eq. (8)),
//                     top-P of the anchor prefix = the bank         (Eq. (13))
//   bank refinement   candidates = the group's bank, then t+1..i    (Eq. (14));
//                     the bank is staged once into LDS
#include "device.h"
#include "launch.h"

namespace dsaidx {

constexpr int kTileKeys = 64;   // keys per pipeline stage: two 32-key MFMA sub-tiles
constexpr int kStageEntries = kSelectHistWords / 2;  // LDS append stage per wave
constexpr int kMaxBankLds = 16384;

template <int DT, int MT, int D, int WPB>
struct ScanCfg {
  static constexpr int kThreads = WPB * 64;
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

// One 64-key tile held in registers between its global load and its LDS store.
template <int NL>
struct TileRegs {
  u32x4 v[NL];
  int tok;   // key index of candidate `tid` of the tile (threads < 64)
  float ks;  // its fp8 scale
};

template <int DT, int MT, int D, bool BANK, int WPB>
__global__ void __launch_bounds__(WPB * 64, 2) scan_topk_kernel(const ScanArgs args) {
  using C = ScanCfg<DT, MT, D, WPB>;
  using Frag = typename AFrag<DT>::type;
  constexpr int kThreads = C::kThreads;
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[3][kTileKeys * C::kLdsRow];
  __shared__ int32_t s_tok[3][kTileKeys];
  __shared__ float s_kscale[3][kTileKeys];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[WPB][kSelectHistWords];
  __shared__ int32_t s_bank[BANK ? kMaxBankLds : 1];
  __shared__ int s_need[3];  // compaction requests of steps i % 3

  const int tid = threadIdx.x;
  // wave-uniform by construction; readfirstlane lets the compiler see it, so
  // every per-query condition below is a scalar branch, not an exec-mask dance
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int h = l >> 5;    // which half of the k range / which 16 of each 32 heads
  const int col = l & 31;  // MFMA column = key within a 32-key sub-tile

  // queries of this workgroup: the longest candidate lists are launched first
  const int j_hi = (int)args.nq - (int)blockIdx.x * WPB - 1;  // highest row
  const int j = j_hi - (WPB - 1) + wave;                      // this wave's row
  const bool active = j >= 0;
  const int j_lo = j_hi - (WPB - 1) < 0 ? 0 : j_hi - (WPB - 1);
  const int pos0 = (int)args.pos0;

  // candidate list of the workgroup
  int bank_len = 0;
  int anchor = 0;
  const int t_hi = pos0 + j_hi * args.pos_stride;
  int ncand_blk;
  if constexpr (BANK) {
    const int grp = j_lo / args.group;  // all WPB rows share one group
    anchor = pos0 + grp * args.group;
    bank_len = min(args.bank_stride, anchor + 1);
    ncand_blk = bank_len + (t_hi - anchor);
    const int32_t* gbank = args.bank + (int64_t)grp * args.bank_stride;
    for (int i = tid; i < bank_len; i += kThreads) s_bank[i] = gbank[i];
    __syncthreads();
  } else {
    ncand_blk = t_hi + 1;
  }
  // candidate c of the workgroup -> key index
  auto cand_token = [&](int c) __attribute__((always_inline)) -> int {
    if constexpr (!BANK) return c;
    return c < bank_len ? s_bank[c] : anchor + 1 + (c - bank_len);
  };
  const int t_me = pos0 + (active ? j : j_lo) * args.pos_stride;
  const int ncand_me = BANK ? bank_len + (t_me - anchor) : t_me + 1;
  const int ntiles = (ncand_blk + kTileKeys - 1) / kTileKeys;

  // ---- this wave's query: A fragments and gate weights in registers
  Frag a[MT][C::kSteps];
  float wv[MT][16];
  {
    float qs = 1.0f;
    if (DT == kFP8 && active) qs = args.q_scale[j];
    const int jq = active ? j : 0;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int head = 32 * m + col;
      const bool hv = active && head < args.H;
      const uint8_t* qrow =
          (const uint8_t*)args.q + ((int64_t)jq * args.H + (hv ? head : 0)) * C::kRowBytes;
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
        wv[m][r] = (active && hr < args.H) ? args.w[(int64_t)jq * args.H + hr] * qs : 0.0f;
      }
    }
  }

  uint32_t* ckey = args.cand_key + (int64_t)(active ? j : 0) * args.cap;  // raw fp32 scores
  int32_t* cidx = args.cand_idx + (int64_t)(active ? j : 0) * args.cap;
  uint32_t* hist = s_hist[wave];
  // Scores that enter are first staged in this wave's LDS (the selection
  // histogram's words, free outside a selection) and flushed to the global
  // buffer in order when the stage nears full: the tile loop then issues few
  // global stores.  A flush does not wait for its stores (a wait would drain
  // the tile prefetches queued before them on the same in-order counter);
  // they are waited for only where the buffer is read back.
  uint32_t* stage_key = hist;
  int32_t* stage_idx = (int32_t*)(hist + kStageEntries);
  int cnt = 0;                       // entries in the global buffer (wave-uniform)
  int nst = 0;                       // entries in the LDS stage (wave-uniform)
  float thr = -__builtin_inff();     // scores must exceed this to enter (wave-uniform)
  auto flush = [&]() __attribute__((always_inline)) {
    for (int e = l; e < nst; e += 64) {
      ckey[cnt + e] = stage_key[e];
      cidx[cnt + e] = stage_idx[e];
    }
    cnt += nst;
    nst = 0;
  };
  // A wave whose buffer passes `lim` raises the flag of the current step; after
  // that step's barrier every wave holding more than K entries compacts, so the
  // workgroup pays for one selection at a time instead of one per wave.  A
  // step appends at most 64 entries, so the buffer cannot overflow meanwhile.
  const int lim = args.cap - 192;  // cnt + nst <= lim + 64 < cap after a step
  if (tid < 3) s_need[tid] = 0;

  // ---- tile pipeline: global -> registers (3 sets) -> LDS (3 stages).  Tile t
  // is loaded at step t-4, stored to LDS stage t%3 at step t-2 and scored at
  // step t; its first sub-tile's MFMAs are issued at the end of step t-1.
  using Regs = TileRegs<C::kLoads>;
  // Loads are unconditional (candidates past the end read the last valid
  // row; their scores are masked when appended), so no load sits behind a
  // branch and the register ring's wait counts stay exact.
  auto load_tile = [&](Regs& R, int it) __attribute__((always_inline)) {
    const int base = it * kTileKeys;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int c = (tid + i * kThreads) % C::kChunks;
      const int r = c / C::kChunksPerRow, p = c % C::kChunksPerRow;
      const int tok = cand_token(min(base + r, ncand_blk - 1));
      R.v[i] = *(const u32x4*)((const uint8_t*)args.k + (int64_t)tok * C::kRowBytes + p * 16);
    }
    const int tok = cand_token(min(base + (tid & (kTileKeys - 1)), ncand_blk - 1));
    R.tok = tok;
    if constexpr (DT == kFP8) R.ks = args.k_scale[tok];
  };
  auto store_tile = [&](const Regs& R, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int c = tid + i * kThreads;
      if (c < C::kChunks) {
        const int r = c / C::kChunksPerRow, p = c % C::kChunksPerRow;
        *(u32x4*)(&s_tile[buf][r * C::kLdsRow + p * 16]) = R.v[i];
      }
    }
    if (tid < kTileKeys) {
      s_tok[buf][tid] = R.tok;
      if constexpr (DT == kFP8) s_kscale[buf][tid] = R.ks;
    }
  };

  // MFMAs of 32-key sub-tile u of the tile in LDS stage `buf`
  auto mfma_sub = [&](v16f (&acc)[MT], int buf, int u) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = v16f{};
    const uint8_t* brow = &s_tile[buf][(32 * u + col) * C::kLdsRow + h * C::kHalf];
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      Frag b;
      if constexpr (DT == kBF16) {
        b = __builtin_bit_cast(v8bf, *(const u32x4*)(brow + 16 * s));
      } else {
        struct { u32x4 lo, hi; } pr = {*(const u32x4*)(brow + 32 * s),
                                       *(const u32x4*)(brow + 32 * s + 16)};
        b = __builtin_bit_cast(v8i, pr);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = mfma<DT>(a[m][s], b, acc[m]);
    }
  };
  // ReLU + gate-weighted head sum (Eq. (1)) of this lane's 16*MT heads
  auto head_sum = [&](const v16f (&acc)[MT]) __attribute__((always_inline)) -> float {
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m) gated_relu_sum16(wv[m], acc[m], s0, s1);
    return s0 + s1;
  };
  // the full score of sub-tile u's key in this lane's column; the other
  // 16*MT heads of that key live in lane l ^ 32, so after the swap both lane
  // halves hold the sum.  A negative sum times a zero key scale is -0, which
  // the ranking treats as +0: adding +0 turns it into +0.
  auto sub_score = [&](float part, int buf, int u) __attribute__((always_inline)) -> float {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false,
                                               false);
    float sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if constexpr (DT == kFP8) sc *= s_kscale[buf][32 * u + col];
    return sc + 0.0f;
  };
  // append the step's scores that beat the threshold: lane l holds candidate
  // tbase + l (sub-tile 0 in the low lane half, sub-tile 1 in the high half),
  // so lane order is candidate order and one ballot serves 64 candidates
  auto append = [&](float sc, int buf, int tbase, int step_buf) __attribute__((always_inline)) {
    uint64_t tm = ballot(sc > thr);
    if (tbase + kTileKeys > ncand_me) tm &= ballot(tbase + l < ncand_me);  // the query's last tile
    if (tm) {
      if ((tm >> l) & 1) {
        const int p = nst + rank_below(tm);
        stage_key[p] = __float_as_uint(sc);
        stage_idx[p] = BANK ? s_tok[buf][l] : tbase + l;
      }
      nst += popc(tm);
      if (cnt + nst > lim && l == 0) s_need[step_buf] = 1;
    }
  };
  // interleave the next sub-tile's MFMAs with the current head sums
  constexpr int kNumMfma = MT * C::kSteps;
  constexpr int kValuPerMfma = (32 * MT + kNumMfma - 1) / kNumMfma;
  auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < kNumMfma; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
    }
  };

  Regs R0, R1, R2;
  v16f acc0[MT], acc1[MT];
  if (ntiles > 0) {
    load_tile(R0, 0);
    load_tile(R1, min(1, ntiles - 1));
    store_tile(R0, 0);
    store_tile(R1, 1);
    load_tile(R2, min(2, ntiles - 1));
    load_tile(R0, min(3, ntiles - 1));
  }
  __syncthreads();
  if (active && ncand_me > 0 && ntiles > 0) mfma_sub(acc0, 0, 0);
  // step i: store tile i+2 (set (i+2)%3), load tile i+4 (into set (i+1)%3),
  // score tile i with tile i+1's first MFMAs in flight
  // `buf` = i % 3, passed as a literal so every LDS address is base + constant
  auto step = [&](Regs& Rs, Regs& Rl, int i, const int buf) __attribute__((always_inline)) {
    const int buf1 = buf == 2 ? 0 : buf + 1, buf2 = buf == 0 ? 2 : buf - 1;
    // requests raised during step i-1 (seen after its barrier); clear the
    // flag of step i+1, last read before the previous barrier
    if (i > 0 && s_need[buf2] && active && cnt + nst > args.K) {
      flush();
      wave_mem_fence();  // the buffer's stores land before the selection reads it
      thr = wave_select_topk(ckey, cidx, cnt, args.K, hist);
      cnt = args.K;
    } else if (active && nst > kStageEntries - 64) {
      flush();
    }
    if (tid == 0) s_need[buf1] = 0;
    // the same loads and LDS stores every step (past the last tile they
    // repeat it and are never read), so the wait counts are exact
    store_tile(Rs, buf2);
    load_tile(Rl, min(i + 4, ntiles - 1));
    const int tbase = i * kTileKeys;
    const bool s0 = active && tbase < ncand_me;
    const bool s1 = active && tbase + 32 < ncand_me;
    const bool n0 = active && tbase + kTileKeys < ncand_me && i + 1 < ntiles;
    float sc0 = 0.0f, sc1 = 0.0f;
    if (s0) {
      float part;
      if (s1) {
        mfma_sub(acc1, buf, 1);
        part = head_sum(acc0);
        interleave();
      } else {
        part = head_sum(acc0);
      }
      sc0 = sub_score(part, buf, 0);
    }
    if (s1) {
      float part;
      if (n0) {
        mfma_sub(acc0, buf1, 0);
        part = head_sum(acc1);
        interleave();
      } else {
        part = head_sum(acc1);
      }
      sc1 = sub_score(part, buf, 1);
    } else if (n0) {
      mfma_sub(acc0, buf1, 0);
    }
    if (s0) append(l < 32 ? sc0 : sc1, buf, tbase, buf);
    __syncthreads();
  };
  for (int i = 0; i < ntiles; i += 3) {
    step(R2, R1, i, 0);
    if (i + 1 < ntiles) step(R0, R2, i + 1, 1);
    if (i + 2 < ntiles) step(R1, R0, i + 2, 2);
  }

  if (!active) return;
  flush();
  wave_emit_topk<16>(ckey, cidx, cnt, args.K, hist, args.out_idx + (int64_t)j * args.out_stride,
                     args.out_score ? args.out_score + (int64_t)j * args.out_stride : nullptr);
}

template <int DT, int MT, int D, bool BANK, int WPB>
static hipError_t launch_bw(const ScanArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.nq + WPB - 1) / WPB;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((scan_topk_kernel<DT, MT, D, BANK, WPB>), dim3((unsigned)blocks),
                     dim3(WPB * 64), 0, stream, a);
  return hipGetLastError();
}

// 8 queries per workgroup; 4 when bank groups of 4 must not straddle a workgroup
template <int DT, int MT, int D>
static hipError_t launch_t(const ScanArgs& a, hipStream_t stream) {
  if (!a.bank) return launch_bw<DT, MT, D, false, 8>(a, stream);
  if (a.group % 8 == 0) return launch_bw<DT, MT, D, true, 8>(a, stream);
  return launch_bw<DT, MT, D, true, 4>(a, stream);
}

hipError_t launch_scan_topk(const ScanArgs& a, int dtype, hipStream_t stream) {
  if (dense_topk_supported(a)) return launch_dense_topk(a, dtype, stream);
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
