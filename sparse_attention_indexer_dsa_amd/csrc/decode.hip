// decode.hip -- decode-time indexer for gfx950: one new bf16 query per
// sequence scores its whole E4M3 key cache (ADIndex (Qi et al.), Section 3:
// O(L) work per decoding query), then the top-K of each row (Eq. (2)).
//
// decode_scan: the cache stream is the cost.  A workgroup walks a span of up
// to 16384 keys of one row, 768 keys per loop trip; each wavefront takes 32
// keys at a time, lane l loading its key's k-half (d/2 bytes) straight into
// registers (four 32-key tiles in flight while two others are scored), widens
// E4M3 to bf16 exactly (every E4M3 value is a bf16 value) with
// v_cvt_scalef32_pk_bf16_fp8, and runs the bf16 MFMA with the query's heads on
// M.  ReLU, the gate-weighted head sum and the per-key scale follow in
// registers.  Scores stay in LDS together with a histogram of the top 12 bits
// of their order-preserving keys; the histogram is added to the row's, and
// only the scores in bins at or above the bin of the span's own K-th best (a
// lower bound of the row's K-th best) leave the chip, as a compact list whose
// four segments the four waves write in one pass.  HBM writes cost far more
// than their share of the traffic, so the row of scores is never written
// whole.
//
// Selection, with the row histogram's bin b* that holds the row's K-th best:
//   decode_classify (one workgroup per span): counts the span's list entries
//     above b* and gathers those inside b* into the row's candidate array;
//   decode_select (one workgroup per row): two radix rounds over the
//     candidates in LDS find the exact K-th score and the tie cut (ties:
//     lower index first), and a prefix sum gives every span's output offset;
//   decode_emit (one workgroup per span): writes the span's selected keys in
//     ascending index at that offset.
// Rows of at most K keys are written by decode_select from the lists; rows
// whose b* bin is too crowded take an exact multi-pass path over the lists.
#include "device.h"
#include "launch.h"

namespace dsaidx {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecTilesPerTrip = 6;  // per wave: three pairs of 32-key tiles
static_assert(kDecKeysPerPass == kDecWaves * kDecTilesPerTrip * 32, "one loop trip = 6 tiles per wave");

// ------------------------------------------------------------------ select

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Exclusive prefix sum over a workgroup of NW waves (all threads call);
// `total` gets the sum.
template <int NW = kSelWaves>
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int& total) {
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int incl = wave_incl_scan(v);
  if (l == 63) s_tmp[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
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
template <int NW = kSelWaves, typename F>
__device__ __forceinline__ void block_find_digit(int per, F bins, int krem, int* s_tmp,
                                                 int* s_res) {
  const int tid = threadIdx.x;
  int local = 0;
  for (int i = 0; i < per; ++i) local += bins(tid, i);
  int total;
  const int excl = block_excl_scan<NW>(local, s_tmp, total);
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

template <int D>
struct DecTile {
  static constexpr int kVec = D / 2 / 16;  // 16-byte loads per lane per tile
  u32x4 v[kVec];
};

// R rows per workgroup (R > 1: 8 heads each, one shared key source): the R
// queries' heads fill 8R rows of the same MFMAs, so the keys are read once
// for all of them; each row keeps its own score stage, histogram and lists.
template <int MT, int D, int R>
__global__ void __launch_bounds__(kDecThreads, 2) decode_scan_kernel(const DecodeArgs args) {
  static_assert(R == 1 || MT == 1, "several rows per workgroup share one 32-row MFMA tile");
  constexpr int kSteps = D / 16;  // bf16 k-steps
  constexpr int kHalf = D / 2;    // fp8 bytes of a lane's k-half
  constexpr int kVec = DecTile<D>::kVec;
  constexpr int kStageKeys = dec_max_kpb(R);
  __shared__ uint32_t s_hist[R][kDecHistBins / 2];  // two 16-bit counts per word
  __shared__ float s_score[R][kStageKeys];
  __shared__ int s_tmp[kDecWaves];
  __shared__ int s_res[4];
  const int rg = blockIdx.y;  // rows rg*R .. rg*R + R-1
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = tid & 63;
  const int h = l >> 5, col = l & 31;
  const int64_t blk0 = (int64_t)blockIdx.x * args.kpb;
  int span_r[R];  // keys of each row inside this workgroup's span
  int64_t n = 0;  // the longest row
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t nr = args.seq_lens[rg * R + r];
    nr = nr < 0 ? 0 : (nr > args.Nmax ? args.Nmax : nr);
    n = nr > n ? nr : n;
    const int64_t left_r = nr - blk0;
    span_r[r] = left_r <= 0 ? 0 : (int)(left_r < args.kpb ? left_r : args.kpb);
  }
  if (blk0 >= n) return;
  // loop trips of this workgroup: 768 keys each, none wholly past the row end
  const int64_t left = n - blk0 < args.kpb ? n - blk0 : args.kpb;
  const int trips = (int)((left + kDecKeysPerPass - 1) / kDecKeysPerPass);
  for (int i = tid; i < R * kDecHistBins / 2; i += kDecThreads) (&s_hist[0][0])[i] = 0;

  // the R rows' queries are consecutive in q [rows, H, d] and w [rows, H]:
  // together they are one query of R*H heads
  const int HR = R * args.H;
  v8bf a[MT][kSteps];
  float wv[MT][16];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int head = 32 * m + col;
    const bool hv = head < HR;
    const uint8_t* qrow =
        (const uint8_t*)args.q + ((int64_t)rg * HR + (hv ? head : 0)) * (2 * D);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      u32x4 v = hv ? *(const u32x4*)(qrow + h * D + 16 * s) : u32x4{0, 0, 0, 0};
      a[m][s] = __builtin_bit_cast(v8bf, v);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hr = 32 * m + 8 * (r >> 2) + 4 * h + (r & 3);
      wv[m][r] = hr < HR ? args.w[(int64_t)rg * HR + hr] : 0.0f;
    }
  }
  __syncthreads();

  // Buffer resources over this workgroup's span [blk0, blk_end) of the row:
  // the hardware range check returns zeros for loads past the span, so no
  // load sits behind a branch and the load-counter waits in the loop stay
  // exact.  Scores are staged in LDS and written out after the loop, so the
  // loop issues no global stores at all.
  const int64_t blk_end = n < blk0 + args.kpb ? n : blk0 + args.kpb;
  const int span = (int)(blk_end - blk0);
  const int b0 = rg * R;  // the row whose key source the workgroup reads
  const uint8_t* kc_row = args.row_kc ? args.row_kc[b0] : args.kc + (int64_t)b0 * args.Nmax * D;
  const float* ks_row = args.row_ks ? args.row_ks[b0] : args.k_scale + (int64_t)b0 * args.Nmax;
  const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kc_row + blk0 * D), (short)0, span * D, kBufferWord3);
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ks_row + blk0), (short)0, span * 4, kBufferWord3);

  // tile i of this wave covers span keys (i*kDecWaves + wave)*32 + [0, 32)
  auto key_of = [&](int i) __attribute__((always_inline)) { return (i * kDecWaves + wave) * 32 + col; };
  auto load = [&](DecTile<D>& t, float& ks, int i) __attribute__((always_inline)) {
    const int key = key_of(i);
#pragma unroll
    for (int v = 0; v < kVec; ++v)
      t.v[v] = __builtin_amdgcn_raw_buffer_load_b128(kres, key * D + h * kHalf + 16 * v, 0, 0);
    ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sres, key * 4, 0, 0));
  };
  auto score = [&](const DecTile<D>& t, float ks, int i) __attribute__((always_inline)) {
    const int key = key_of(i);
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
    // row r's heads are MFMA rows 8r .. 8r+7: accumulators 4r .. 4r+3 of
    // this lane (heads 4h .. 4h+3 of the row); R == 1 sums every head
    constexpr int kAcc = R == 1 ? 16 : 4;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float s0 = 0.0f, s1 = 0.0f;
      if constexpr (R == 1) {
#pragma unroll
        for (int m = 0; m < MT; ++m) gated_relu_sum16(wv[m], acc[m], s0, s1);
      } else {
#pragma unroll
        for (int i = kAcc * r; i < kAcc * (r + 1); i += 2) {
          s0 = fmaf(wv[0][i], relu_bits(acc[0][i]), s0);
          s1 = fmaf(wv[0][i + 1], relu_bits(acc[0][i + 1]), s1);
        }
      }
      float sc = s0 + s1;
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc), false,
                                                 false);
      sc = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * ks;
      sc += 0.0f;  // -0 -> +0
      // lanes l and l+32 hold the same key: the low half records it
      if (l < 32 && key < span_r[r]) {
        s_score[r][key] = sc;
        const uint32_t bin = order_key(sc) >> (32 - kDecHistBits);
        atomicAdd(&s_hist[r][bin >> 1], 1u << (16 * (bin & 1)));
      }
    }
  };

  // Tiles go in pairs through a ring of three pair slots: while one pair is
  // scored the loads of the next two pairs are in flight (16 KB per wave).
  // Scheduling barriers keep the loads in program order, so each wait is for
  // the pair about to be scored and never for the pairs behind it.
  DecTile<D> ta0, ta1, tb0, tb1, tc0, tc1;
  float ka0, ka1, kb0, kb1, kc0, kc1;
  auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
  load(ta0, ka0, 0);
  load(ta1, ka1, 1);
  fence();
  load(tb0, kb0, 2);
  load(tb1, kb1, 3);
  fence();
  for (int i = 0; i < kDecTilesPerTrip * trips; i += kDecTilesPerTrip) {
    load(tc0, kc0, i + 4);
    load(tc1, kc1, i + 5);
    fence();
    score(ta0, ka0, i);
    score(ta1, ka1, i + 1);
    fence();
    load(ta0, ka0, i + 6);
    load(ta1, ka1, i + 7);
    fence();
    score(tb0, kb0, i + 2);
    score(tb1, kb1, i + 3);
    fence();
    load(tb0, kb0, i + 8);
    load(tb1, kb1, i + 9);
    fence();
    score(tc0, kc0, i + 4);
    score(tc1, kc1, i + 5);
    fence();
  }
  __syncthreads();
  for (int r = 0; r < R; ++r) {
    const int b = rg * R + r;
    const int span_b = span_r[r];
    if (span_b == 0) continue;  // the row ends before this span
    uint32_t* hst = s_hist[r];
    const float* scr = s_score[r];
    uint32_t* ghist = args.hist + (int64_t)b * kDecHistBins;
    for (int i = tid; i < kDecHistBins / 2; i += kDecThreads) {
      const uint32_t c = hst[i];
      if (c & 0xFFFFu) atomicAdd(ghist + 2 * i, c & 0xFFFFu);
      if (c >> 16) atomicAdd(ghist + 2 * i + 1, c >> 16);
    }
    // The K-th best score of the span is a lower bound of the row's K-th
    // best: scores below it cannot reach the row's top K and are not kept.
    // The list keeps every score in the histogram bin that holds it or above
    // (a finer cut took a second pass over the span, which cost more than
    // the longer lists do downstream).  A span of at most K keys keeps
    // everything.
    uint32_t keep_from = 0;  // keep scores with (order key >> 8) >= keep_from
    if (span_b > args.K) {
      constexpr int kPer = kDecHistBins / kDecThreads;
      auto bins16 = [&](int t, int i) __attribute__((always_inline)) {
        const int bin = t * kPer + i;
        return (int)((hst[bin >> 1] >> (16 * (bin & 1))) & 0xFFFFu);
      };
      block_find_digit<kDecWaves>(kPer, bins16, args.K, s_tmp, s_res);
      const uint32_t bloc = (uint32_t)s_res[0];
      keep_from = bloc << 12;
    }
    // compact list of the kept scores: wave w writes segment w, the kept
    // keys of the span's w-th quarter in ascending order, 64 consecutive keys
    // per step (lane l key base + l: conflict-free LDS reads), eight LDS reads
    // in flight per lane, in one pass.  Kept entries gather in a per-wave LDS
    // stage (the histogram's words, free now) and leave it 64 at a time, so
    // every list store but the last writes a whole wave's 256 bytes.
    static_assert(kDecListSegs == kDecWaves, "one list segment per wave");
    static_assert(kDecHistBins / 2 >= kDecWaves * 256, "a 128-entry stage per wave");
    const int seg = (int)args.kpb / kDecListSegs;
    const int c0 = wave * seg, c1 = c0 + seg < span_b ? c0 + seg : span_b;
    const int64_t sbase = ((int64_t)b * args.nblk + blockIdx.x) * args.kpb + c0;
    __syncthreads();  // every wave is done with the histogram's words
    uint32_t* stg_sc = hst + wave * 256;                  // score bits [128]
    int32_t* stg_ix = (int32_t*)(hst + wave * 256 + 128);  // key indices [128]
    int pos = 0, nst = 0;  // wave-uniform: entries written, entries staged (< 64 between steps)
    for (int base = c0; base < c1; base += 8 * 64) {
      uint32_t kk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = base + 64 * u + l;
        kk[u] = e < c1 ? order_key(scr[e]) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = base + 64 * u + l;
        const bool keep = e < c1 && (kk[u] >> 8) >= keep_from;
        const uint64_t km = ballot(keep);
        if (keep) {
          const int p = nst + rank_below(km);
          stg_sc[p] = __float_as_uint(key_to_float(kk[u]));
          stg_ix[p] = (int32_t)(blk0 + e);
        }
        nst += popc(km);
        if (nst >= 64) {  // a whole wave's worth: store it, keep the rest
          wave_lds_sync();
          args.cl_sc[sbase + pos + l] = __uint_as_float(stg_sc[l]);
          args.cl_idx[sbase + pos + l] = stg_ix[l];
          const uint32_t rs = stg_sc[64 + l];
          const int32_t ri = stg_ix[64 + l];
          wave_lds_sync();
          if (l < nst - 64) {
            stg_sc[l] = rs;
            stg_ix[l] = ri;
          }
          pos += 64;
          nst -= 64;
          wave_lds_sync();
        }
      }
    }
    wave_lds_sync();
    if (l < nst) {
      args.cl_sc[sbase + pos + l] = __uint_as_float(stg_sc[l]);
      args.cl_idx[sbase + pos + l] = stg_ix[l];
    }
    pos += nst;
    if (l == 0) args.cl_cnt[((int64_t)b * args.nblk + blockIdx.x) * kDecListSegs + wave] = pos;
    if (R > 1) __syncthreads();  // s_tmp, s_res and the histogram serve the next row
  }
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

constexpr int kShift = 32 - kDecHistBits;  // order key -> histogram bin

// Exclusive prefix over the workgroup of N counts at once (one round of
// barriers for all N): before[n] = sum of lower threads' v[n], total[n] = sum.
template <int N>
__device__ __forceinline__ void block_excl_scan_n(const int (&v)[N], int (&before)[N], int (&total)[N],
                                                  int* s_tmp) {
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  int incl[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    incl[n] = wave_incl_scan(v[n]);
    if (l == 63) s_tmp[n * kSelWaves + wave] = incl[n];
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < N; ++n) {
    int b = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      const int t = s_tmp[n * kSelWaves + w];
      b += w < wave ? t : 0;
      all += t;
    }
    before[n] = b + incl[n] - v[n];
    total[n] = all;
  }
  __syncthreads();
}

// Exact multi-pass selection over a row's compact lists in global memory
// (rows whose threshold bin or whose flat list is too long for the finish pass).
// The lists hold every score that can reach the top K, in ascending key order,
// and sit side by side: list j of the row is slots j*kpb .. j*kpb + c_j - 1 of
// one array, so a pass walks all slots in order, kIter batches at a time, with
// kIter 16-byte loads in flight per thread.  In batch k, thread t holds slots
// 4t .. 4t+3 of the batch, so (batch, thread, slot) is key order.
constexpr int kIter = 4;
__device__ void select_lists_exact(const DecodeArgs& args, int b, int nb, uint32_t bstar, int need,
                                   int32_t* oidx, float* osc, uint32_t* s_h, int* s_tmp, int* s_res,
                                   int* s_tmpn, int* s_cnt) {
  const int tid = threadIdx.x;
  const int K = args.K;
  constexpr int kB = 4 * kSelThreads;  // slots per batch
  const int64_t row0 = (int64_t)b * args.nblk * args.kpb;
  const int64_t nslots = (int64_t)nb * args.kpb;
  const int seg = (int)args.kpb / kDecListSegs;  // slots per list segment
  const int nseg = nb * kDecListSegs;
  const int64_t cbase = (int64_t)b * args.nblk * kDecListSegs;
  for (int j = tid; j < nseg && j < kSelThreads; j += kSelThreads) s_cnt[j] = args.cl_cnt[cbase + j];
  __syncthreads();
  // segment j's entry count (segments past the LDS copy are read from memory)
  auto count = [&](uint32_t j) __attribute__((always_inline)) {
    return j < (uint32_t)kSelThreads ? s_cnt[j] : args.cl_cnt[cbase + j];
  };
  auto load = [&](int64_t s0, float (&v)[kIter][4], uint32_t (&ok)[kIter]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kIter; ++k) {
      const int64_t s = s0 + k * kB + 4 * tid;  // a segment is a multiple of 4 slots
      const uint32_t su = (uint32_t)s;              // slots of a row fit in 32 bits
      const int lim = s < nslots ? count(su / (uint32_t)seg) - (int)(su % (uint32_t)seg) : 0;
      ok[k] = lim >= 4 ? 0xFu : (lim > 0 ? (1u << lim) - 1u : 0u);
      if (s < nslots) {
        const v4f a = *(const v4f*)(args.cl_sc + row0 + s);
#pragma unroll
        for (int u = 0; u < 4; ++u) v[k][u] = a[u];
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[k][u] = 0.0f;
      }
    }
  };
  // the row histogram already fixed the top 12 bits of the K-th key (bin b*)
  // and how many of b*'s keys are selected: two 10-bit rounds finish it
  uint32_t prefix = bstar << kShift, pmask = ~0u << kShift;
  int krem = need;
  for (int round = 0; round < 2; ++round) {
    const int shift = round == 0 ? 10 : 0;
    constexpr int nbins = 1024;
    const uint32_t dmask = (uint32_t)nbins - 1;
    for (int i = tid; i < nbins; i += kSelThreads) s_h[i] = 0;
    __syncthreads();
    for (int64_t s0 = 0; s0 < nslots; s0 += kIter * kB) {
      float v[kIter][4];
      uint32_t ok[kIter];
      load(s0, v, ok);
#pragma unroll
      for (int k = 0; k < kIter; ++k)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t key = order_key(v[k][u]);
          if ((ok[k] >> u & 1u) && (key & pmask) == prefix) atomicAdd(&s_h[(key >> shift) & dmask], 1u);
        }
    }
    __syncthreads();
    block_find_digit(1, [&](int t, int i) { return (int)s_h[t + i]; }, krem, s_tmp, s_res);
    prefix |= (uint32_t)s_res[0] << shift;
    pmask |= dmask << shift;
    krem = s_res[1];
    __syncthreads();
  }
  const uint32_t kth = prefix;
  const int keep_eq = krem;  // keys equal to kth: keep the keep_eq lowest indices
  // ordered emission
  int out = 0, eq_seen = 0;
  for (int64_t s0 = 0; s0 < nslots; s0 += kIter * kB) {
    float v[kIter][4];
    uint32_t ok[kIter];
    load(s0, v, ok);
    int nq[kIter], qb[kIter], qt[kIter];
    uint32_t eqm[kIter], gtm[kIter];
#pragma unroll
    for (int k = 0; k < kIter; ++k) {
      eqm[k] = gtm[k] = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t key = order_key(v[k][u]);
        if (ok[k] >> u & 1u) {
          eqm[k] |= (uint32_t)(key == kth) << u;
          gtm[k] |= (uint32_t)(key > kth) << u;
        }
      }
      nq[k] = __builtin_popcount(eqm[k]);
    }
    block_excl_scan_n<kIter>(nq, qb, qt, s_tmpn);
    int nk[kIter], kb[kIter], kt[kIter];
    uint32_t keep[kIter];
    int eq_base = eq_seen;
#pragma unroll
    for (int k = 0; k < kIter; ++k) {
      int eq = eq_base + qb[k];
      keep[k] = gtm[k];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (eqm[k] >> u & 1u) {
          if (eq < keep_eq) keep[k] |= 1u << u;
          ++eq;
        }
      }
      nk[k] = __builtin_popcount(keep[k]);
      eq_base += qt[k];
    }
    block_excl_scan_n<kIter>(nk, kb, kt, s_tmpn);
    int base = out;
#pragma unroll
    for (int k = 0; k < kIter; ++k) {
      if (keep[k]) {
        // the key indices of this thread's kept slots: one 16-byte load
        const int64_t s = s0 + k * kB + 4 * tid;
        const u32x4 ix = *(const u32x4*)(args.cl_idx + row0 + s);
        int p = base + kb[k];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (keep[k] >> u & 1u) {
            if (p < K) {
              oidx[p] = (int32_t)ix[u];
              if (osc) osc[p] = v[k][u];
            }
            ++p;
          }
        }
      }
      base += kt[k];
    }
    out = base;
    eq_seen = eq_base;
  }
}


constexpr int kSpanThreads = 256;
constexpr int kSpanWaves = kSpanThreads / 64;

// Threshold bin b* of row b from its histogram (all threads of the workgroup
// call): s_res[0] = b*, s_res[1] = entries of b* inside the top K, s_res[2] =
// entries in b*.  Thread t holds bins [t*per, (t+1)*per), read as 16-byte
// vectors in one round trip.
template <int NW>
__device__ __forceinline__ void row_threshold(const DecodeArgs& args, int b, int* s_tmp, int* s_res) {
  constexpr int kPer = kDecHistBins / (NW * 64);
  static_assert(kPer % 4 == 0, "whole 16-byte vectors of bins per thread");
  const int tid = threadIdx.x;
  const u32x4* src = (const u32x4*)(args.hist + (int64_t)b * kDecHistBins + tid * kPer);
  uint32_t c[kPer];
#pragma unroll
  for (int q = 0; q < kPer / 4; ++q) {
    const u32x4 v = src[q];
    c[4 * q] = v[0];
    c[4 * q + 1] = v[1];
    c[4 * q + 2] = v[2];
    c[4 * q + 3] = v[3];
  }
  int local = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) local += (int)c[i];
  int total;
  const int excl = block_excl_scan<NW>(local, s_tmp, total);
  const int above = total - excl - local;  // entries in higher threads' (higher) bins
  const int krem = args.K;
  if (above < krem && above + local >= krem) {
    int acc = above;
    bool found = false;
#pragma unroll
    for (int i = kPer - 1; i >= 0; --i) {
      if (!found && acc + (int)c[i] >= krem) {
        s_res[0] = tid * kPer + i;
        s_res[1] = krem - acc;
        s_res[2] = (int)c[i];
        found = true;
      }
      acc += (int)c[i];
    }
  }
  __syncthreads();
}

// List entries a span workgroup loads per thread at once (strided by the
// workgroup size, so every load is coalesced and all of them are in flight).
constexpr int kSpanBatch = 16;

// The compact list of span j of row b read as one list, its segments in
// order (ascending keys): entry e of the list sits at slot(e).
struct SpanList {
  int64_t base;  // the span's first slot
  int seg;       // slots per segment
  int p1, p2, p3, n;  // entries before segments 1, 2, 3; entries in all
  __device__ __forceinline__ SpanList(const DecodeArgs& a, int b, int j) {
    static_assert(kDecListSegs == 4, "four segments per list");
    const int64_t sp = (int64_t)b * a.nblk + j;
    base = sp * a.kpb;
    seg = (int)a.kpb / kDecListSegs;
    const int32_t* c = a.cl_cnt + sp * kDecListSegs;
    p1 = c[0];
    p2 = p1 + c[1];
    p3 = p2 + c[2];
    n = p3 + c[3];
  }
  __device__ __forceinline__ int64_t slot(int e) const {
    const int w = (e >= p1) + (e >= p2) + (e >= p3);
    const int before = w == 0 ? 0 : (w == 1 ? p1 : (w == 2 ? p2 : p3));
    return base + (int64_t)w * seg + (e - before);
  }
};

// One workgroup per (span, row): counts the span's list entries above b* and
// gathers those inside b* into the row's candidate array.
__global__ void __launch_bounds__(kSpanThreads) decode_classify_kernel(const DecodeArgs args) {
  __shared__ int s_tmp[kSpanWaves];
  __shared__ int s_res[4];
  __shared__ int s_base;
  const int b = blockIdx.y, j = blockIdx.x;
  const int tid = threadIdx.x;
  // the span's list counts are read together with the row's length (they lie
  // inside the workspace for every span of the grid; unused past the row)
  const SpanList L(args, b, j);
  int64_t n = args.seq_lens[b];
  n = n < 0 ? 0 : (n > args.Nmax ? args.Nmax : n);
  if (n <= args.K || (int64_t)j * args.kpb >= n) return;
  const int c = L.n;
  // the first batch of the list (scores and key indices together, so a
  // candidate's index needs no second round trip) is requested before the
  // threshold search
  uint32_t key[kSpanBatch];
  int32_t kid[kSpanBatch];
  auto load_batch = [&](int base) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kSpanBatch; ++u) {
      const int e = base + u * kSpanThreads + tid;
      const int64_t sl = e < c ? L.slot(e) : 0;
      key[u] = e < c ? order_key(args.cl_sc[sl]) : 0u;  // key 0: below every bin b*
      kid[u] = e < c ? args.cl_idx[sl] : 0;
    }
  };
  load_batch(0);
  row_threshold<kSpanWaves>(args, b, s_tmp, s_res);
  const uint32_t bstar = (uint32_t)s_res[0];
  if (s_res[2] > kDecCandCap) return;  // the select pass takes the exact path
  uint32_t* ck = args.cand_key + (int64_t)b * kDecCandCap;
  int32_t* ci = args.cand_idx + (int64_t)b * kDecCandCap;
  int above = 0;
  for (int base = 0; base < c; base += kSpanBatch * kSpanThreads) {
    if (base > 0) load_batch(base);
    int cand = 0;
#pragma unroll
    for (int u = 0; u < kSpanBatch; ++u) {
      above += (key[u] >> kShift) > bstar;
      cand += (key[u] >> kShift) == bstar && key[u] != 0u;
    }
    int tot;
    const int before = block_excl_scan<kSpanWaves>(cand, s_tmp, tot);
    if (tot == 0) continue;
    if (tid == 0) s_base = atomicAdd(args.cand_cnt + b, tot);
    __syncthreads();
    int p = s_base + before;
#pragma unroll
    for (int u = 0; u < kSpanBatch; ++u) {
      if ((key[u] >> kShift) == bstar && key[u] != 0u) {
        if (p < kDecCandCap) {
          ck[p] = key[u];
          ci[p] = kid[u];
        }
        ++p;
      }
    }
    __syncthreads();  // s_base is rewritten by the next batch
  }
  int tot_above;
  block_excl_scan<kSpanWaves>(above, s_tmp, tot_above);
  if (tid == 0) args.span_above[(int64_t)b * args.nblk + j] = tot_above;
}

// One workgroup per row: the exact K-th key among the candidates of b*, the
// tie cut, and every span's output offset.  Rows of at most K keys, and rows
// whose b* bin or span count is too large, are written here completely.
static_assert(kSelThreads <= kDecCandCap, "each thread's first candidate slot is inside the row's array");
__global__ void __launch_bounds__(kSelThreads) decode_select_kernel(const DecodeArgs args) {
  __shared__ uint32_t s_ckey[kDecCandCap];
  __shared__ int32_t s_cidx[kDecCandCap];
  __shared__ uint32_t s_h[2048];
  __shared__ int s_tmp[kSelWaves];
  __shared__ int s_res[4 + 2 * kSelWaves];
  __shared__ int s_chosen[kSelThreads];  // chosen candidates per span
  __shared__ int s_tmpn[kIter * kSelWaves];
  __shared__ int s_cnt[kSelThreads];  // list entries per span (exact path)
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  // reads that depend on nothing, issued together before the first wait: the
  // row's candidate count, each thread's first candidate and its span's
  // count above b* (all inside the workspace, whatever the row needs)
  const int nc = args.cand_cnt[b];
  const uint32_t ck0 = args.cand_key[(int64_t)b * kDecCandCap + tid];
  const int32_t ci0 = args.cand_idx[(int64_t)b * kDecCandCap + tid];
  const int above0 = tid < args.nblk ? args.span_above[(int64_t)b * args.nblk + tid] : 0;
  int64_t n = args.seq_lens[b];
  if (args.skip_negative && n < 0) return;  // a row this launch does not own
  n = n < 0 ? 0 : (n > args.Nmax ? args.Nmax : n);
  const int K = args.K;
  int32_t* oidx = args.out_idx + (int64_t)b * K;
  float* osc = args.out_score ? args.out_score + (int64_t)b * K : nullptr;
  const int nb = (int)((n + args.kpb - 1) / args.kpb);  // scan spans of the row
  if (tid == 0) args.rowsel[4 * b] = 0;  // written here unless set below
  if (n <= K) {
    // every span kept all of its keys: the lists are keys 0 .. n-1 in order
    int off = 0;
    for (int j = 0; j < nb; ++j) {
      const SpanList L(args, b, j);
      for (int i = tid; i < L.n; i += kSelThreads) {
        const int64_t sl = L.slot(i);
        oidx[off + i] = args.cl_idx[sl];
        if (osc) osc[off + i] = args.cl_sc[sl];
      }
      off += L.n;
    }
    for (int p = (int)n + tid; p < K; p += kSelThreads) {
      oidx[p] = -1;
      if (osc) osc[p] = -__builtin_inff();
    }
    return;
  }
  row_threshold<kSelWaves>(args, b, s_tmp, s_res);
  const uint32_t bstar = (uint32_t)s_res[0];
  const int need = s_res[1];     // entries of bin b* that are selected
  const int in_bin = s_res[2];   // keys of the row in bin b* (the histogram's count)
  __syncthreads();
  if (in_bin > kDecCandCap || nb > kSelThreads) {  // the same test decode_classify made
    select_lists_exact(args, b, nb, bstar, need, oidx, osc, s_h, s_tmp, s_res, s_tmpn, s_cnt);
    return;
  }
  // The candidates are the list entries in b*: every span keeps whole bins
  // from its own K-th best's bin up, which is at most b*, so b*'s keys are all
  // listed (the count is at most in_bin either way, and a key a list did not
  // keep could not be selected).
  if (tid < nc) {
    s_ckey[tid] = ck0;
    s_cidx[tid] = ci0;
  }
  for (int i = tid + kSelThreads; i < nc; i += kSelThreads) {
    s_ckey[i] = args.cand_key[(int64_t)b * kDecCandCap + i];
    s_cidx[i] = args.cand_idx[(int64_t)b * kDecCandCap + i];
  }
  s_chosen[tid] = 0;
  __syncthreads();

  // exact K-th key among the candidates (the low 20 bits, two rounds)
  uint32_t prefix = bstar << kShift, pmask = ~0u << kShift;
  int krem = need;
  block_radix_lds(s_ckey, nc, 10, 1024, prefix, pmask, krem, s_h, s_tmp, s_res);
  const int n_eq = block_radix_lds(s_ckey, nc, 0, 1024, prefix, pmask, krem, s_h, s_tmp, s_res);
  const uint32_t kth = prefix;
  const int keep_eq = krem;  // of the n_eq candidates equal to kth keep the keep_eq lowest indices
  // ties at kth: the keep_eq-th largest ~index among them is the cut
  uint32_t idx_cut = 0u;  // selected: key > kth, or key == kth and ~index >= idx_cut
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
      const int pb = (nbins + kSelThreads - 1) / kSelThreads;
      block_find_digit(pb, [&](int t, int i) { return t * pb + i < nbins ? (int)s_h[t * pb + i] : 0; },
                       tk, s_tmp, s_res);
      tp |= (uint32_t)s_res[0] << shift;
      tm |= dmask << shift;
      tk = s_res[1];
      __syncthreads();
    }
    idx_cut = tp;
  }
  // chosen candidates per span, then each span's output offset
  for (int i = tid; i < nc; i += kSelThreads) {
    const uint32_t key = s_ckey[i];
    const uint32_t e = (uint32_t)s_cidx[i];
    if (key > kth || (key == kth && ~e >= idx_cut)) atomicAdd(&s_chosen[e / (uint32_t)args.kpb], 1);
  }
  __syncthreads();
  const int mine = tid < nb ? s_chosen[tid] + above0 : 0;  // nb <= nblk
  int total;
  const int off = block_excl_scan(mine, s_tmp, total);
  if (tid < nb) args.span_off[(int64_t)b * args.nblk + tid] = off;
  if (tid == 0) {
    args.rowsel[4 * b + 1] = kth;
    args.rowsel[4 * b + 2] = idx_cut;
    args.rowsel[4 * b] = 1;
  }
}

// One workgroup per (span, row): writes the span's selected keys, in
// ascending index, at the span's output offset.  Entry base + u*256 + tid sits
// in thread tid's register u; a prefix over the (u, wave) ballot counts orders
// the writes.
__global__ void __launch_bounds__(kSpanThreads) decode_emit_kernel(const DecodeArgs args) {
  __shared__ int s_tmp[kSpanWaves];
  __shared__ int s_wc[kSpanBatch * kSpanWaves];
  const int b = blockIdx.y, j = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  // the row's length and selection, and the span's list counts and output
  // offset, are independent reads: all are issued before the first test
  const SpanList L(args, b, j);
  const int sel_mode = args.rowsel[4 * b];
  const uint32_t kth = args.rowsel[4 * b + 1], idx_cut = args.rowsel[4 * b + 2];
  const int off0 = args.span_off[(int64_t)b * args.nblk + j];
  int64_t n = args.seq_lens[b];
  n = n < 0 ? 0 : (n > args.Nmax ? args.Nmax : n);
  if ((int64_t)j * args.kpb >= n || sel_mode != 1) return;
  const int c = L.n;
  int32_t* oidx = args.out_idx + (int64_t)b * args.K;
  float* osc = args.out_score ? args.out_score + (int64_t)b * args.K : nullptr;
  int out = off0;
  for (int base = 0; base < c; base += kSpanBatch * kSpanThreads) {
    float v[kSpanBatch];
    int32_t idx[kSpanBatch];
#pragma unroll
    for (int u = 0; u < kSpanBatch; ++u) {
      const int e = base + u * kSpanThreads + tid;
      const int64_t sl = e < c ? L.slot(e) : 0;
      v[u] = e < c ? args.cl_sc[sl] : 0.0f;
      idx[u] = e < c ? args.cl_idx[sl] : -1;
    }
    bool sel[kSpanBatch];
#pragma unroll
    for (int u = 0; u < kSpanBatch; ++u) {
      const uint32_t key = order_key(v[u]);
      sel[u] = idx[u] >= 0 && (key > kth || (key == kth && ~(uint32_t)idx[u] >= idx_cut));
      const int cnt = popc(ballot(sel[u]));
      if (l == 0) s_wc[u * kSpanWaves + wave] = cnt;
    }
    __syncthreads();
    int total;
    const int vwc = tid < kSpanBatch * kSpanWaves ? s_wc[tid] : 0;
    const int before = block_excl_scan<kSpanWaves>(vwc, s_tmp, total);
    if (tid < kSpanBatch * kSpanWaves) s_wc[tid] = before;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSpanBatch; ++u) {
      const int pos = out + s_wc[u * kSpanWaves + wave] + rank_below(ballot(sel[u]));
      if (sel[u] && pos < args.K) {
        oidx[pos] = idx[u];
        if (osc) osc[pos] = v[u];
      }
    }
    out += total;
    __syncthreads();  // s_wc is rewritten by the next batch
  }
}

template <int MT, int D>
static hipError_t launch_dec(const DecodeArgs& a, hipStream_t stream) {
  if (a.B <= 0) return hipSuccess;
  // histograms and candidate counters are contiguous: one fill clears both
  hipError_t e = launch_fill_i32((int32_t*)a.hist, (int64_t)a.B * kDecHistBins + a.B, 0, stream);
  if (e != hipSuccess) return e;
  const int R = a.scan_rows > 1 ? a.scan_rows : 1;
  if (a.nblk > 0) {
    const dim3 grid((unsigned)a.nblk, (unsigned)(a.B / R));
    if constexpr (MT == 1) {
      if (R == 2)
        hipLaunchKernelGGL((decode_scan_kernel<1, D, 2>), grid, dim3(kDecThreads), 0, stream, a);
      else if (R == 4)
        hipLaunchKernelGGL((decode_scan_kernel<1, D, 4>), grid, dim3(kDecThreads), 0, stream, a);
      else
        hipLaunchKernelGGL((decode_scan_kernel<1, D, 1>), grid, dim3(kDecThreads), 0, stream, a);
    } else {
      hipLaunchKernelGGL((decode_scan_kernel<MT, D, 1>), grid, dim3(kDecThreads), 0, stream, a);
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.nblk > 0)
    hipLaunchKernelGGL(decode_classify_kernel, dim3((unsigned)a.nblk, (unsigned)a.B), dim3(kSpanThreads), 0,
                       stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_select_kernel, dim3((unsigned)a.B), dim3(kSelThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.nblk > 0)
    hipLaunchKernelGGL(decode_emit_kernel, dim3((unsigned)a.nblk, (unsigned)a.B), dim3(kSpanThreads), 0, stream,
                       a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.scan_rows > 1 && (!dec_scan_rows_ok(a.scan_rows, a.H, a.B) || !a.row_kc || !a.row_ks ||
                          a.kpb > dec_max_kpb(a.scan_rows)))
    return hipErrorInvalidValue;
  const int MT = a.H <= 32 ? 1 : 2;
  if (MT == 1) {
    if (a.d == 64) return launch_dec<1, 64>(a, stream);
    return launch_dec<1, 128>(a, stream);
  }
  if (a.d == 64) return launch_dec<2, 64>(a, stream);
  return launch_dec<2, 128>(a, stream);
}

// p[0, n) = v: 16-byte stores from the first 16-byte boundary, single words
// before it and after the last whole vector.
__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t head = (int64_t)((16u - ((uintptr_t)p & 15u)) & 15u) / 4;  // words before the boundary
  const int64_t h = head < n ? head : n;
  const int64_t nq = (n - h) / 4;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, stride = (int64_t)gridDim.x * blockDim.x;
  u32x4* q = (u32x4*)(p + h);
  const u32x4 vv = {(uint32_t)v, (uint32_t)v, (uint32_t)v, (uint32_t)v};
  for (int64_t i = t0; i < nq; i += stride) q[i] = vv;
  if (t0 < h) p[t0] = v;
  if (t0 < n - h - 4 * nq) p[h + 4 * nq + t0] = v;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n / 4 + 255) / 256 + 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

}  // namespace dsaidx
