// dense_topk.hip -- the dense causal indexer for 33..64 heads at d = 128 on
// gfx950: score + streaming top-K per query (ADIndex (Qi et al.), Section 3,
// Eq. (1) and Eq. (2)), the layout the long-context prefill runs in.
//
// One wavefront owns one query (at position pos0 + j * pos_stride) and walks
// its candidate keys 0..t in ascending index; the 8 waves of a workgroup own 8
// consecutive queries and share one stream of key tiles: 128 keys for E4M3
// over contiguous keys, 64 for bf16 (twice the bytes per key) and for
// gathering.
//
//   * Tiles go from HBM straight into a five-stage LDS ring with
//     global_load_lds (no register staging): tile t is requested four steps
//     before it is scored, into stage t % 5.  Each lane's 16-byte chunk lands
//     at lane*16 of the wave's 1 KB; lanes fetch the chunks of each key row in
//     an order XOR-swizzled by the row index, so the MFMA operand reads are
//     free of bank conflicts without padding.
//   * Per-head dot products: fp8 v_mfma_f32_32x32x64_f8f6f4 or bf16
//     v_mfma_f32_32x32x16_bf16, heads on M (two 32-row tiles), keys on N,
//     fp32 accumulation; B operands are read from LDS one 32-key sub-tile
//     ahead of their MFMAs.
//   * ReLU through the identity w*ReLU(s) = (w/2)*|s| + (w/2)*s: the first
//     term is one FMA with an |.| source modifier per (head, key), the second
//     summed over heads is (sum_j (w_j/2) q_j) . k, a single dot product per
//     (query, key) that the workgroup computes with 16x16x32 MFMAs.  Its
//     query vector q~ is split into parts that the MFMA takes exactly:
//     bf16 keys use three bf16 parts (24 significant bits); E4M3 keys use an
//     fp16 high and low part (22 bits) of q~ times a power of two that puts
//     its largest element just below 2^15, undone after the product (every
//     E4M3 value is exact in fp16, every bf16 value in bf16).  The linear
//     term then carries about fp32's own rounding (integer-valued inputs stay
//     exact), which keeps scores near zero, where the two terms cancel,
//     within the tolerance.
//   * Streaming top-K exactly as the general kernel: scores that beat the
//     running threshold are staged in LDS, flushed to the query's candidate
//     buffer, and compacted by a wave radix select when it fills (two 11-bit
//     digits, and the third only when the K-th best's 22-bit key bucket is
//     crowded); keys arrive in ascending index, so strict ">" keeps the lower
//     index on ties.
//   * Full-row top-K, for launches whose rows all fit their buffer (cap at
//     least the largest row's candidate count): each 64 scores go to their
//     candidate slots with one buffer store (the buffer range
//     drops those past the row) and counts them in the wave's LDS histogram
//     of the top 11 key bits.  Nothing is appended or compacted; at the end
//     the histogram gives the first radix digit, one pass over the row keeps
//     the entries at or above that digit's bin (with their key positions)
//     and counts the second digit, and the third digit and the output pass
//     run over the kept list.
//   * Gathering (the bank refinement of Eq. (14), groups of a multiple of 8
//     queries): the workgroup's candidates are its group's bank followed by
//     the keys after the anchor.  Each tile's 64 bank positions are copied
//     into an eight-slot LDS ring seven steps ahead; the tile requests read
//     them and fetch the listed rows (and fp8 scales) with the same LDS DMA,
//     and the append stores positions instead of list slots.  The list is
//     ascending in position, so ties still keep the lower index.
//   * Sampled start (contiguous keys; E4M3 rows of 16K candidates and more,
//     bf16 rows of 12K and more): a pre-pass of the same kernel scores, per
//     workgroup, one or two rounds of the ring of sample keys spread evenly
//     over its shortest row and gives each query a start that about 3.5 K of
//     its keys beat (the 16-bit key bucket of its m-th best sample).  The
//     stream then keeps only scores above the start, so far fewer enter the
//     buffer and it is compacted about once instead of four times.  The top
//     K all lie above the start whenever at least K entries did; the stream
//     checks that at its end, and a query that kept fewer writes nothing and
//     flags its workgroup (the pre-pass cleared the flag); a third launch
//     streams the flagged workgroups again from -inf (every other workgroup
//     of it ends at once), so the result never depends on the sample.  The
//     start leaves at least 35 samples expected above it, which makes a flag
//     rarer than one query in 10^9 on i.i.d. scores.  The stream's own code
//     is the same with or without a start.  Shorter bf16 rows gain nothing:
//     the pre-pass repeats the prologue (each query's 16 KB of fragments).
#include "device.h"
#include "launch.h"

namespace dsaidx {

namespace {

constexpr int kTile = 64;       // keys per append (one 64-lane ballot); the bf16 and gathering step
constexpr int kStages = 5;      // LDS ring stages
constexpr int kAhead = 4;       // a tile is requested this many steps before it is scored
constexpr int kWaves = 8;       // queries per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kStage = kSelectHistWords / 2;  // LDS append stage entries per wave
constexpr int kD = 128;
constexpr int kIdxRing = 8;   // gathering: tiles of bank positions held in LDS
constexpr int kIdxAhead = 7;  // a tile's positions are requested this many steps before it is scored
// sampled start: the shortest row that samples (E4M3, bf16), the fewest
// samples a query expects above its start, and the radix digits of the
// start's select over the samples' 16-bit keys (a 9-bit digit, then the low
// 9 bits)
constexpr int kSampleMinRowFp8 = 16384;
constexpr int kSampleMinRowBf16 = 12288;
constexpr int sample_min_row(int dt) { return dt == kFP8 ? kSampleMinRowFp8 : kSampleMinRowBf16; }
constexpr int kSampleMinAbove = 35;
constexpr int kSampleBins = 512;

// The rank m of a query's sampled start among its S samples.  If the samples
// fell like independent draws, mu = K S / n of them would beat the row's K-th
// best score, and the start fails (fewer than K keys beat it) only when at
// least m of them do: m = min(3.5 mu, mu + 6 sqrt(mu) + 10) + 1 puts that
// binomial tail below 5e-10 wherever m >= 35 (the least that sampling takes),
// while the share of the row kept above the start falls from 3.5 K to under
// 2 K once mu reaches about 80.
__device__ __forceinline__ int64_t start_rank(int K, int64_t S, int64_t n) {
  const float mu = (float)K * (float)S / (float)n;
  return (int64_t)fminf(3.5f * mu, mu + 6.0f * __builtin_sqrtf(mu) + 10.0f) + 1;
}

template <int S>
struct StageC {  // a ring stage as a compile-time constant
  constexpr operator int() const { return S; }
};

template <bool B>
struct SampleC {  // whether a step scores sample keys, as a compile-time constant
  static constexpr bool value = B;
};

template <int DT, int TK>
struct Cfg {
  static constexpr int kRowBytes = DT == kBF16 ? 2 * kD : kD;
  static constexpr int kTileBytes = TK * kRowBytes;
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kDma = kTileBytes / (kThreads * 16);  // 16-byte DMAs per lane per tile
  static constexpr int kSteps = DT == kBF16 ? kD / 16 : kD / 64;  // main MFMA k-steps
  // vm operations a wave issues per step: the tile chunks and the key scales
  // (one 64-lane request per 64 keys)
  static constexpr int kVmPerStep = kDma + TK / 64;
  // chunk c of row r sits at slot c ^ swz(r): any 16 consecutive rows then put
  // a given chunk in 16 distinct 16-byte bank groups (a 16-lane LDS pass)
  static __device__ __forceinline__ int swz(int r) { return DT == kBF16 ? (r & 15) : ((r >> 1) & 7); }
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

typedef __attribute__((address_space(3))) void lds_void;
typedef int v4i __attribute__((ext_vector_type(4)));

// Descriptor words of a raw buffer of `bytes` bytes at p (no stride; reads
// past the end return zero), held in SGPRs.
__device__ __forceinline__ v4i raw_buffer_words(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  v4i r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = (int)kBufferWord3;
  return r;
}

// LDS byte address of a pointer into a __shared__ array (wave-uniform here).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)p);
}

// Tile loads straight into LDS (buffer_load ... lds): lane i's bytes land at
// LDS address m0 + size * i.  They are written as asm, not with the builtin,
// because the compiler cannot tell the LDS stage a builtin load writes from
// the stages the same step reads (the stage index is a run-time value), and so
// it waits for every load in flight, this step's too, before each LDS read: the
// ring's prefetch distance collapses to zero.  The kernel orders the ring
// itself: a wave waits for its own loads of a tile with s_waitcnt vmcnt and the
// barrier that follows publishes the tile to the workgroup.  These loads have
// no register results, so nothing is left in flight that the compiler could
// reuse.  The compiler writes m0 (an operand bound to it); the leading wait
// state covers the SALU-write-of-m0 to LDS-DMA hazard, which the compiler
// cannot see inside asm.
__device__ __forceinline__ void dma_b128(const v4i& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma_b32(const v4i& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// SAMPLE: the sampled start's pre-pass (E4M3 over contiguous keys): the
// sample tiles only, then each query's start into args.start.
template <int DT, bool GATHER, bool FULL, bool SAMPLE>
__global__ void __launch_bounds__(kThreads, 2) dense_topk_kernel(const ScanArgs args) {
  // keys per step: E4M3 scores 128 keys (four 32-key sub-tiles) between
  // barriers, so the step's fixed costs (the compaction check, the waits and
  // the barrier) are paid once per 128 keys; bf16 tiles are twice the bytes
  // and keep 64, as does gathering
  constexpr int TK = (DT == kFP8 && !GATHER) ? 128 : 64;
  constexpr int kHalves = TK / 64;  // 64-key halves of a tile (one append each)
  using C = Cfg<DT, TK>;
  // vm operations a wave issues per step: the tile chunks, the key scales and,
  // gathering, the candidate indices of a later tile
  constexpr int kVm = C::kVmPerStep + (GATHER ? 1 : 0);
  using Frag = typename AFrag<DT>::type;
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[kStages][C::kTileBytes];
  __shared__ float s_ks[kStages][TK];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[kWaves][kSelectHistWords];
  // the linear terms of a tile: [slot][d half][query][key], slot = the tile's
  // ring stage, or (128-key tiles) its parity: tile t+1's are written while
  // tile t's are read
  constexpr int kLinSlots = TK == 128 ? 2 : kStages;
  __shared__ float s_lin[kLinSlots][2][kWaves][TK];
  // parts of q-tilde: bf16 hi / mid / lo (bf16 keys) or scaled fp16 hi / lo
  // (E4M3 keys), and the factor that undoes the fp16 parts' scale
  constexpr int kParts = DT == kBF16 ? 3 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t s_qt[kWaves][kParts][kD];
  __shared__ float s_qinv[kWaves];
  __shared__ int s_need[2];  // s_need[i & 1] == i: a wave asked for compaction in step i
  // gathering: the bank positions of tiles t .. t+7, slot t & 7 (tile t+7's
  // are requested in step t, read by tile t+4's request and tile t's append)
  __shared__ int32_t s_idx[GATHER ? kIdxRing : 1][kTile];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int h = l >> 5;    // which half of the k range / which 16 of each 32 heads
  const int col = l & 31;  // MFMA column = key within a 32-key sub-tile

  // queries of this workgroup: the longest candidate lists are launched first
  const int j_hi = (int)args.nq - (int)blockIdx.x * kWaves - 1;
  const int j = j_hi - (kWaves - 1) + wave;
  const bool active = j >= 0;
  const int jq = active ? j : 0;
  const int pos0 = (int)args.pos0;
  const int t_hi = pos0 + j_hi * args.pos_stride;  // the workgroup's last query position
  // Contiguous: the candidates of query t are keys 0 .. t.  Gathering (bank
  // refinement, Eq. (14)): the workgroup's 8 queries belong to one group whose
  // candidates are its bank (nbank ascending positions <= anchor) and then the
  // keys anchor+1 .. t; candidate c is a position either way, ascending.
  int anchor = 0, nbank = 0;
  const int32_t* bank = nullptr;
  if constexpr (GATHER) {
    const int g = (j_hi - (kWaves - 1)) / args.group;
    anchor = pos0 + g * args.group;
    nbank = min(args.bank_stride, anchor + 1);
    bank = args.bank + (int64_t)g * args.bank_stride;
  }
  const int ncand_blk = GATHER ? nbank + (t_hi - anchor) : t_hi + 1;
  const int ncand_me = !active ? 0 : GATHER ? nbank + (pos0 + j - anchor) : pos0 + j * args.pos_stride + 1;
  const int ntiles = (ncand_blk + TK - 1) / TK;
  // Sampled start.  The stream (E4M3 over contiguous keys) takes its query's
  // start from args.start when given; its re-stream launch (args.rerun_pass)
  // runs only the workgroups that the first stream flagged, from -inf.
  constexpr bool kCertify = !GATHER && !FULL && !SAMPLE;
  static_assert(!SAMPLE || (!GATHER && !FULL), "the pre-pass is for streaming rows over contiguous keys");
  if constexpr (kCertify) {
    if (args.rerun_pass && args.rerun[blockIdx.x] == 0) return;
  }
  // The pre-pass: nsamp sample tiles (one or two rounds of the ring), sample
  // s at key s * sstride + sstride / 2, all inside the workgroup's shortest
  // row.  A query's start is its m-th best sample (start_rank: m is about
  // 3.5 K S / ncand + 1 of the S samples for short or few samples, less
  // above); the round count is the least that gives every query of the
  // workgroup m >= kSampleMinAbove.  Workgroups whose rows are short, or
  // whose 3.5 K best keys reach back past key 0, start at -inf.
  int nsamp = 0, sstride = 1;
  if constexpr (SAMPLE) {
    if (tid == 0) args.rerun[blockIdx.x] = 0;  // the stream sets it when a query fails its check
    const int lo = pos0 + max(j_hi - (kWaves - 1), 0) * args.pos_stride + 1;
    if (lo >= sample_min_row(DT) && 7 * (int64_t)args.K < 2 * (int64_t)lo) {
      for (int r = 1; r <= 2 && nsamp == 0; ++r) {
        const int64_t S = (int64_t)r * kStages * TK;
        if (start_rank(args.K, S, ncand_blk) >= kSampleMinAbove) nsamp = r * kStages;
      }
    }
    if (nsamp == 0) {
      if (active) args.start[j] = -__builtin_inff();
      return;
    }
    sstride = lo / (nsamp * TK);
  }

  // ---- this wave's query: A fragments, gate weights (w/2, with the fp8 query
  // scale folded in), and q-tilde = sum_j (w_j/2) q_j split into bf16 hi + lo
  Frag a[2][C::kSteps];
  float wv[2][16];
  {
    const float qs = (DT == kFP8 && active) ? args.q_scale[jq] : 1.0f;
    const float* wrow = args.w + (int64_t)jq * args.H;
    // Every load here is unconditional, with the head clamped into the
    // query's rows and the value zeroed afterwards, and is issued before its
    // first use: behind a branch each load cost the wave a full memory round
    // trip, about a hundred of them before the first tile.
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int head = 32 * m + col;
      const bool hv = active && head < args.H;
      const uint8_t* qrow =
          (const uint8_t*)args.q + ((int64_t)jq * args.H + min(head, args.H - 1)) * C::kRowBytes;
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) {
        if constexpr (DT == kBF16) {
          const u32x4 v = *(const u32x4*)(qrow + h * kD + 16 * s);
          a[m][s] = __builtin_bit_cast(v8bf, hv ? v : u32x4{0, 0, 0, 0});
        } else {
          const u32x4 v0 = *(const u32x4*)(qrow + h * 64 + 32 * s);
          const u32x4 v1 = *(const u32x4*)(qrow + h * 64 + 32 * s + 16);
          struct { u32x4 lo, hi; } pr = {hv ? v0 : u32x4{0, 0, 0, 0}, hv ? v1 : u32x4{0, 0, 0, 0}};
          a[m][s] = __builtin_bit_cast(v8i, pr);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int hr = 32 * m + 8 * (r >> 2) + 4 * h + (r & 3);
        const float wl = wrow[min(hr, args.H - 1)];
        wv[m][r] = (active && hr < args.H) ? 0.5f * wl * qs : 0.0f;
      }
    }
    // q-tilde: lane l owns elements 2l and 2l+1; heads in batches of 16
    // whose loads are all in flight together, summed in head order
    float t0 = 0.0f, t1 = 0.0f;
    if (active) {
      const uint8_t* qb = (const uint8_t*)args.q + (int64_t)jq * args.H * C::kRowBytes;
      constexpr int kB = 16;
      for (int h0 = 0; h0 < args.H; h0 += kB) {
        uint32_t qv[kB];
        float wq[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          const int hd = min(h0 + u, args.H - 1);
          if constexpr (DT == kBF16) qv[u] = *(const uint32_t*)(qb + (int64_t)hd * C::kRowBytes + 4 * l);
          else qv[u] = *(const uint16_t*)(qb + (int64_t)hd * C::kRowBytes + 2 * l);
          wq[u] = wrow[hd];
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          if (h0 + u >= args.H) break;
          const float wh = 0.5f * wq[u] * qs;
          float x0, x1;
          if constexpr (DT == kBF16) {
            x0 = __uint_as_float(qv[u] << 16);
            x1 = __uint_as_float(qv[u] & 0xFFFF0000u);
          } else {
            const v2bf p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qv[u], 1.0f, false);
            x0 = (float)p[0];
            x1 = (float)p[1];
          }
          t0 = fmaf(wh, x0, t0);
          t1 = fmaf(wh, x1, t1);
        }
      }
    }
    if constexpr (DT == kBF16) {
      // three bf16 parts; each remainder is exact in fp32
      float r0 = t0, r1 = t1;
#pragma unroll
      for (int pt = 0; pt < 3; ++pt) {
        const uint16_t b0 = bf16_rne(r0), b1 = bf16_rne(r1);
        s_qt[wave][pt][2 * l] = b0;
        s_qt[wave][pt][2 * l + 1] = b1;
        r0 -= __uint_as_float((uint32_t)b0 << 16);
        r1 -= __uint_as_float((uint32_t)b1 << 16);
      }
    } else {
      // fp16 hi + lo of q-tilde * 2^e, with the query's largest |element|
      // scaled into [2^14, 2^15) (e = 0 for an all-zero q-tilde)
      float mx = fmaxf(__builtin_fabsf(t0), __builtin_fabsf(t1));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      int e = 0;
      if (mx > 0.0f) e = min(15 - __builtin_amdgcn_frexp_expf(mx), 120);
      const float y0 = __builtin_ldexpf(t0, e), y1 = __builtin_ldexpf(t1, e);
      const _Float16 a0 = (_Float16)y0, a1 = (_Float16)y1;
      const _Float16 b0 = (_Float16)(y0 - (float)a0), b1 = (_Float16)(y1 - (float)a1);
      s_qt[wave][0][2 * l] = __builtin_bit_cast(uint16_t, a0);
      s_qt[wave][0][2 * l + 1] = __builtin_bit_cast(uint16_t, a1);
      s_qt[wave][1][2 * l] = __builtin_bit_cast(uint16_t, b0);
      s_qt[wave][1][2 * l + 1] = __builtin_bit_cast(uint16_t, b1);
      if (l == 0) s_qinv[wave] = __builtin_ldexpf(1.0f, -e);
    }
  }

  // ---- the linear-term MFMA of this wave: keys 16*nb .. +15 of a tile, the
  // d half kh (k-steps 2kh, 2kh+1 of 32), all 8 queries on M: row m is part
  // m & 1 (hi, mid / lo) of query m >> 1.  bf16 adds a second MFMA into the
  // same accumulator whose even rows hold the queries' third parts and whose
  // odd rows are zero, so every query's parts still end in rows 2q, 2q+1.
  const int nb = wave & 3, kh = wave >> 2;
  __syncthreads();
  typedef _Float16 v8h __attribute__((ext_vector_type(8)));
  // A fragment of part row m for k-step s (part 2: even rows only)
  auto qt_frag = [&](int part, int s) __attribute__((always_inline)) -> u32x4 {
    const int m = l & 15;
    const u32x4 v = *(const u32x4*)&s_qt[m >> 1][part == 2 ? 2 : (m & 1)][32 * (2 * kh + s) + 8 * (l >> 4)];
    return (part == 2 && (m & 1)) ? u32x4{0u, 0u, 0u, 0u} : v;
  };
  u32x4 la[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) la[s] = qt_frag(0, s);
  const float qinv = DT == kFP8 ? s_qinv[wave] : 1.0f;

  uint32_t* ckey = args.cand_key + (int64_t)jq * args.cap;  // raw fp32 scores
  int32_t* cidx = args.cand_idx + (int64_t)jq * args.cap;
  uint32_t* hist = s_hist[wave];
  // Full-row mode (every candidate list fits a row buffer, cap >= the
  // workgroup's candidates): candidate c's score goes to ckey[c] and into the
  // wave's LDS histogram of the top 11 order-key bits; nothing is appended or
  // compacted, and the histogram gives the final selection its first digit.
  // The row's stores go through a buffer range that drops those past the
  // query's candidates, so every step issues exactly one store.
  const __amdgpu_buffer_rsrc_t rres =
      __builtin_amdgcn_make_buffer_rsrc((void*)ckey, (short)0, FULL ? ncand_me * 4 : 0, kBufferWord3);
  if constexpr (FULL) {
    hist_zero<2048>(hist);
    wave_lds_sync();
  }

  // Scores that enter are staged in this wave's LDS (the selection histogram's
  // words, free outside a selection) and flushed to the candidate buffer when
  // the stage nears full.  A flush does not wait for its stores: the wait is
  // where the buffer is read back.
  uint32_t* stage_key = hist;
  int32_t* stage_idx = (int32_t*)(hist + kStage);
  int cnt = 0;                                        // entries in the buffer
  int nst = 0;                                        // entries in the LDS stage
  // scores must exceed thr: the query's sampled start, when it has one
  float thr = !active ? __builtin_inff()
            : (kCertify && args.start != nullptr && !args.rerun_pass) ? args.start[jq] : -__builtin_inff();
  auto flush = [&]() __attribute__((always_inline)) {
    for (int e = l; e < nst; e += 64) {
      ckey[cnt + e] = stage_key[e];
      cidx[cnt + e] = stage_idx[e];
    }
    cnt += nst;
    nst = 0;
  };
  // A wave whose buffer passes `lim` records the step in s_need; after the
  // step's barrier every wave holding more than K entries compacts.  A step
  // appends at most 64 entries, so the buffer cannot overflow meanwhile.
  const int lim = args.cap - 192;
  if (tid < 2) s_need[tid] = -1;

  // ---- tile requests: this lane's chunks of tile t into LDS stage `st`.
  // Buffer resources end after the workgroup's last query position, so rows
  // past it (the last tile's tail, and the tiles requested past the end) read
  // as zeros and are masked when appended; no request needs a clamp or branch.
  const v4i kres = raw_buffer_words(args.k, (t_hi + 1) * C::kRowBytes);
  const v4i sres = DT == kFP8 ? raw_buffer_words(args.k_scale, (t_hi + 1) * 4)
                              : raw_buffer_words(args.w, 256);
  int lane_row[C::kDma];  // the tile row of this lane's chunk
  int lane_off[C::kDma];  // its byte offset inside the row's position (swizzled chunk)
#pragma unroll
  for (int n = 0; n < C::kDma; ++n) {
    const int ci = n * kThreads + wave * 64 + l;  // chunk position in the stage
    const int r = ci / C::kChunksPerRow, cs = ci % C::kChunksPerRow;
    lane_row[n] = r;
    lane_off[n] = 16 * (cs ^ C::swz(r));
  }
  // gathering: the position of candidate c of tile t (past the list: none)
  constexpr uint32_t kNowhere = 0x80000000u;  // an offset past every buffer range (all < 2 GiB)
  auto position = [&](int t, int c) __attribute__((always_inline)) -> int {
    return c < nbank ? s_idx[t & (kIdxRing - 1)][c & (kTile - 1)] : anchor + 1 + (c - nbank);
  };
  // LDS addresses (scalar): this wave's part of stage 0, the scales of stage 0
  const uint32_t lds_tile = lds_addr(&s_tile[0][0]) + wave * 64 * 16;
  const uint32_t lds_ks = lds_addr(&s_ks[0][0]);
  auto request = [&](int t, int st) __attribute__((always_inline)) {
    // contiguous keys: tile t holds keys rb + rs * (0 .. TK-1).  The pre-pass
    // reads the sample tiles; its requests past them point past the buffer
    // range, which fetches nothing.
    int rb = t * TK, rs = 1;
    if constexpr (SAMPLE) {
      rb = t < nsamp ? t * TK * sstride + (sstride >> 1) : t_hi + 1;
      rs = t < nsamp ? sstride : 0;
    }
#pragma unroll
    for (int n = 0; n < C::kDma; ++n) {
      uint32_t off;
      if constexpr (GATHER) {
        // past the list the position exceeds t_hi; so does a bank entry of -1
        const uint32_t pos = (uint32_t)position(t, t * kTile + lane_row[n]);
        off = pos <= (uint32_t)t_hi ? pos * C::kRowBytes + lane_off[n] : kNowhere;
      } else {
        off = (uint32_t)(rb + lane_row[n] * rs) * C::kRowBytes + lane_off[n];
      }
      dma_b128(kres, lds_tile + st * C::kTileBytes + n * kThreads * 16, off);
    }
    // every wave writes the same scales (fp8; bf16 loads placeholder words),
    // 64 per request, so all waves issue the same number of requests per step
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) {
      uint32_t soff = 4 * l;
      if constexpr (DT == kFP8) {
        if constexpr (GATHER) {
          const uint32_t pos = (uint32_t)position(t, t * TK + 64 * hh + l);
          soff = pos <= (uint32_t)t_hi ? 4 * pos : kNowhere;
        } else {
          soff = 4 * (rb + (64 * hh + l) * rs);
        }
      }
      dma_b32(sres, lds_ks + (st * TK + 64 * hh) * 4, soff);
    }
  };
  // gathering: tile t's 64 bank positions into the index ring (every wave
  // writes the same words, so every wave issues the same requests)
  const v4i bres = GATHER ? raw_buffer_words(bank, nbank * 4) : v4i{0, 0, 0, 0};
  const uint32_t lds_idx = lds_addr(&s_idx[0][0]);
  auto request_idx = [&](int t) __attribute__((always_inline)) {
    if constexpr (GATHER) dma_b32(bres, lds_idx + (t & (kIdxRing - 1)) * kTile * 4, 4 * (t * kTile + l));
  };

  // B operands of sub-tile u of the tile in stage st (row 32u + col has the
  // swizzle of row col)
  auto load_b = [&](Frag (&bf)[C::kSteps], int st, int u) __attribute__((always_inline)) {
    const uint8_t* row = &s_tile[st][(32 * u + col) * C::kRowBytes];
    const int x = C::swz(col);
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      if constexpr (DT == kBF16) {
        bf[s] = __builtin_bit_cast(v8bf, *(const u32x4*)(row + 16 * ((8 * h + s) ^ x)));
      } else {
        const int c0 = 4 * h + 2 * s;
        struct { u32x4 lo, hi; } pr = {*(const u32x4*)(row + 16 * (c0 ^ x)),
                                       *(const u32x4*)(row + 16 * ((c0 + 1) ^ x))};
        bf[s] = __builtin_bit_cast(v8i, pr);
      }
    }
  };
  // the k-steps [s0, s1) of a sub-tile's MFMAs (s0 == 0 starts from zero)
  auto mfma_steps = [&](v16f (&acc)[2], const Frag (&bf)[C::kSteps], int s0, int s1)
      __attribute__((always_inline)) {
    if (s0 == 0) {
      acc[0] = v16f{};
      acc[1] = v16f{};
    }
#pragma unroll
    for (int s = s0; s < s1; ++s) {
      acc[0] = mfma<DT>(a[0][s], bf[s], acc[0]);
      acc[1] = mfma<DT>(a[1][s], bf[s], acc[1]);
    }
  };
  auto mfma_sub = [&](v16f (&acc)[2], const Frag (&bf)[C::kSteps]) __attribute__((always_inline)) {
    mfma_steps(acc, bf, 0, C::kSteps);
  };
  // sum over this lane's 32 heads of (w/2)*|s|
  auto abs_sum = [&](const v16f (&acc)[2]) __attribute__((always_inline)) -> float {
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        s0 = fmaf(wv[m][r], __builtin_fabsf(acc[m][r]), s0);
        s1 = fmaf(wv[m][r + 1], __builtin_fabsf(acc[m][r + 1]), s1);
      }
    }
    return s0 + s1;
  };
  // the linear-term slot of tile t (in ring stage st)
  auto lin_slot = [&](int t, int st) __attribute__((always_inline)) { return TK == 128 ? (t & 1) : st; };
  // the linear term of 64-key half hh of tile t (in stage st) for all 8
  // queries: this wave's 16 keys and d half, written to s_lin[slot][kh]
  auto linear = [&](int t, int st, int hh) __attribute__((always_inline)) {
    v4f c = {0.0f, 0.0f, 0.0f, 0.0f};
    const int r = 64 * hh + 16 * nb + (l & 15);
    const uint8_t* row = &s_tile[st][r * C::kRowBytes];
    const int x = C::swz(r);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int ks = 2 * kh + s;  // d elements 32ks + 8(l>>4) .. +7
      if constexpr (DT == kBF16) {
        const v8bf kb = __builtin_bit_cast(v8bf, *(const u32x4*)(row + 16 * ((4 * ks + (l >> 4)) ^ x)));
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, la[s]), kb, c, 0, 0, 0);
        // the third parts, read from LDS here rather than held in registers
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, qt_frag(2, s)), kb, c, 0, 0, 0);
      } else {
        const int d0 = 32 * ks + 8 * (l >> 4);
        const uint2 v = *(const uint2*)(row + 16 * ((d0 >> 4) ^ x) + (d0 & 15));
        const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.x, 1.0f, false);
        const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.x, 1.0f, true);
        const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.y, 1.0f, false);
        const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.y, 1.0f, true);
        const v8h kb = __builtin_bit_cast(
            v8h, u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                       __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)});
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, la[s]), kb, c, 0, 0, 0);
      }
    }
    // rows 4(l>>4)+i = (query 2(l>>4) + i/2, part i%2)
    const int q0 = 2 * (l >> 4);
    const int sl = lin_slot(t, st);
    s_lin[sl][kh][q0][r] = c[0] + c[1];
    s_lin[sl][kh][q0 + 1][r] = c[2] + c[3];
  };
  // the full scores of the step's 64 keys, key l in lane l (sub-tile l / 32,
  // column l % 32).  p0 and p1 hold this lane's half-head sums for its column
  // of sub-tiles 0 and 1; swapping the upper half of p0 with the lower half of
  // p1 leaves both halves of key l's sum in lane l, in the same order on both
  // lane halves (lower-half heads first).  Then the linear term and the fp8
  // key scale: (sum over heads of (w/2)|s| + linear term) * scale.  Adding +0
  // last turns a -0 (a negative sum times a zero scale, or a sum of -0 terms)
  // into +0, which is how the ranking treats it.
  // the LDS terms of key 64*hh + l of tile t: its two half-d linear terms and
  // its fp8 scale (read ahead of the score that needs them)
  struct Terms { float lin0, lin1, ks; };
  auto read_terms = [&](int t, int st, int hh) __attribute__((always_inline)) -> Terms {
    const int sl = lin_slot(t, st), key = 64 * hh + l;
    return Terms{s_lin[sl][0][wave][key], s_lin[sl][1][wave][key], DT == kFP8 ? s_ks[st][key] : 1.0f};
  };
  auto score_of = [&](float p0, float p1, const Terms& tm) __attribute__((always_inline)) -> float {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    // E4M3: the linear term comes scaled by 2^e; qinv = 2^-e undoes it
    float sc = fmaf(tm.lin0 + tm.lin1, qinv, __uint_as_float(sw[0]) + __uint_as_float(sw[1]));
    if constexpr (DT == kFP8) sc *= tm.ks;
    return sc + 0.0f;
  };
  auto tile_score = [&](float p0, float p1, int t, int st, int hh) __attribute__((always_inline)) -> float {
    return score_of(p0, p1, read_terms(t, st, hh));
  };
  // append the step's scores that beat the threshold: lane l holds candidate
  // tbase + l, so lane order is candidate order and one ballot serves 64
  auto append = [&](float sc, int tbase, int i) __attribute__((always_inline)) {
    if constexpr (FULL) {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rres, 4 * (tbase + l), 0, 0);
      if (tbase + l < ncand_me) hist_add<2048>(hist, order_key(sc), 21);
      return;
    }
    uint64_t tm = ballot(sc > thr);
    if (tbase + kTile > ncand_me) tm &= ballot(tbase + l < ncand_me);  // the query's last tile
    if (tm) {
      if ((tm >> l) & 1) {
        const int p = nst + rank_below(tm);
        stage_key[p] = __float_as_uint(sc);
        stage_idx[p] = GATHER ? position(i, tbase + l) : tbase + l;
      }
      nst += popc(tm);
      if (cnt + nst > lim && l == 0) s_need[i & 1] = i;
    }
  };
  // The pre-pass's sample tiles: each score's top 16 order-key bits, in this
  // wave's LDS words past the start's histogram
  uint16_t* const samp = (uint16_t*)(hist + kSampleBins / 2);
  static_assert(2 * kStages * 128 <= 2 * (kSelectHistWords - kSampleBins / 2), "two rounds of samples fit");
  // The start: the 16-bit key of the m-th best of the S samples (two radix
  // digits), taken at the bottom of its bucket so that it errs low; -inf when
  // m leaves too few samples above it or reaches past them.
  auto sampled_start = [&]() __attribute__((always_inline)) -> float {
    const int S = nsamp * TK;
    const int64_t m = start_rank(args.K, S, ncand_me);
    if (m >= S || m < kSampleMinAbove) return -__builtin_inff();
    uint32_t prefix = 0, pmask = 0;
    int krem = (int)m;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = pass == 0 ? 7 : 0;
      hist_zero<kSampleBins>(hist);
      wave_lds_sync();
      for (int e = l; e < S; e += 64) {
        const uint32_t k = samp[e];
        if ((k & pmask) == prefix) hist_add<kSampleBins>(hist, k, shift);
      }
      wave_lds_sync();
      radix_pick<kSampleBins>(hist, shift, prefix, pmask, krem);
      wave_lds_sync();
    }
    // a test hook: a start above every score, so that every sampled query
    // keeps nothing and its workgroup streams again
    if (args.sample_test) return __builtin_inff();
    return key_to_float(prefix << 16);
  };

  // ---- prologue: (gathering: the positions of tiles 0..6) tiles 0..3
  // requested, tile 0's linear term, first MFMAs
  if constexpr (GATHER) {
    for (int t = 0; t < kIdxAhead; ++t) request_idx(t);
    __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): this wave's copy of the positions
    __syncthreads();
  }
  for (int t = 0; t < kAhead; ++t) request(t, t);
  __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): tiles 0..3 in LDS
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < kHalves; ++hh) linear(0, 0, hh);
  v16f acc0[2], acc1[2];
  Frag bA[C::kSteps], bB[C::kSteps];
  load_b(bA, 0, 0);
  mfma_sub(acc0, bA);
  load_b(bB, 0, 1);
  __syncthreads();  // s_lin of tile 0

  // step i scores tile i (stage st = i % 5) while tile i+1 (stage st1) feeds
  // the next MFMAs and its linear term, and tile i+4 is requested into stage
  // st4 = (i+4) % 5, the one tile i-1 left.  On entry bB holds tile i's second
  // sub-tile's B operands and acc0 its first sub-tile's products.  For fp8
  // the loop is unrolled over the ring so that every stage is a constant (LDS
  // addresses fold into the instructions' offsets); bf16, whose operands take
  // twice the registers, keeps one copy of the step with run-time stages.
  auto step = [&](const int i, auto stage, auto sample) __attribute__((always_inline)) {
    constexpr bool kSamp = decltype(sample)::value;  // tile i is a sample tile
    const int st = stage;
    const int st1 = st == kStages - 1 ? 0 : st + 1;
    const int st4 = st == 0 ? kStages - 1 : st - 1;  // (st + kAhead) % kStages
    // compaction requests raised during step i-1 (seen after its barrier)
    if constexpr (!FULL && !kSamp) {
      if (i > 0 && s_need[(i - 1) & 1] == i - 1 && active && cnt + nst > args.K) {
        flush();
        thr = wave_keep_topk(ckey, cidx, cnt, args.K, hist, kCompactSlack);
      } else if (nst > kStage - TK) {
        flush();
      }
    }
    request(i + kAhead, st4);
    request_idx(i + kIdxAhead);
    const int tbase = i * TK;
    // the same work every step: past the last tile the MFMAs run on zeros
    // and the append masks them out
    load_b(bA, st1, 0);
    mfma_sub(acc1, bB);
    const float p0 = abs_sum(acc0);
    load_b(bB, st1, 1);
    // fp8: half of the next sub-tile's MFMAs are held back until after the
    // linear term, so they still run while the wave scores and appends
    constexpr int kHeld = DT == kFP8 ? C::kSteps / 2 : C::kSteps;
    mfma_steps(acc0, bA, 0, kHeld);
    const float p1 = abs_sum(acc1);
    linear(i + 1, st1, 0);
    if constexpr (kHeld < C::kSteps) mfma_steps(acc0, bA, kHeld, C::kSteps);
    const float sc = tile_score(p0, p1, i, st, 0);
    if constexpr (kSamp) samp[i * TK + l] = (uint16_t)(order_key(sc) >> 16);
    else append(sc, tbase, i);
    // tile i+2 (gathering: and the positions of tile i+5) must have landed
    // before the barrier publishes them: after their requests this wave issued
    // those of steps i-1 and i (and maybe a flush's stores, which only makes
    // the count conservative).  In full-row mode each step also ends with
    // one store, and the two after those requests are allowed to be pending.
    __builtin_amdgcn_s_waitcnt(0x3F70 | (2 * kVm + (FULL ? 2 * kHalves : 0)));
    __syncthreads();
  };
  // The 128-key step (E4M3): tile i's four 32-key sub-tiles, with tile i+1's
  // first sub-tile and its linear terms prepared at the end.  On entry acc0
  // holds sub-tile 0's products and bB sub-tile 1's B operands; the MFMAs of
  // each sub-tile run while the head sums of the one before are taken, and
  // each 64-key half is scored and appended as soon as its sums are complete.
  auto step128 = [&](const int i, auto stage, auto sample) __attribute__((always_inline)) {
    constexpr bool kSamp = decltype(sample)::value;  // tile i is a sample tile
    const int st = stage;
    const int st1 = st == kStages - 1 ? 0 : st + 1;
    const int st4 = st == 0 ? kStages - 1 : st - 1;  // (st + kAhead) % kStages
    if constexpr (!FULL && !kSamp) {
      if (i > 0 && s_need[(i - 1) & 1] == i - 1 && active && cnt + nst > args.K) {
        flush();
        thr = wave_keep_topk(ckey, cidx, cnt, args.K, hist, kCompactSlack);
      } else if (nst > kStage - TK) {
        flush();
      }
    }
    request(i + kAhead, st4);
    const int tbase = i * TK;
    // a sample's top 16 key bits, or the append of a row tile's scores
    auto take = [&](float sc, int hh) __attribute__((always_inline)) {
      if constexpr (kSamp) samp[i * TK + 64 * hh + l] = (uint16_t)(order_key(sc) >> 16);
      else append(sc, tbase + 64 * hh, i);
    };
    load_b(bA, st, 2);
    mfma_sub(acc1, bB);                    // sub-tile 1
    const float p0 = abs_sum(acc0);        // sub-tile 0
    load_b(bB, st, 3);
    mfma_sub(acc0, bA);                    // sub-tile 2
    const float p1 = abs_sum(acc1);        // sub-tile 1
    linear(i + 1, st1, 0);
    take(tile_score(p0, p1, i, st, 0), 0);
    load_b(bA, st1, 0);
    mfma_sub(acc1, bB);                    // sub-tile 3
    const float p2 = abs_sum(acc0);        // sub-tile 2
    load_b(bB, st1, 1);
    constexpr int kHeld = C::kSteps / 2;
    mfma_steps(acc0, bA, 0, kHeld);        // tile i+1, sub-tile 0 (half)
    const float p3 = abs_sum(acc1);        // sub-tile 3
    linear(i + 1, st1, 1);
    mfma_steps(acc0, bA, kHeld, C::kSteps);
    take(tile_score(p2, p3, i, st, 1), 1);
    // tile i+2 must have landed before the barrier publishes it: after its
    // requests this wave issued those of steps i-1 and i; in full-row mode
    // each step also ends with two stores
    __builtin_amdgcn_s_waitcnt(0x3F70 | (2 * kVm + (FULL ? 2 * kHalves : 0)));
    __syncthreads();
  };
  static_assert(kStages == 5 && kAhead == kStages - 1, "the loops below assume a five-stage ring");
  if constexpr (SAMPLE) {
    // nsamp is a whole number of rounds of the ring (bf16, whose fragments
    // take twice the registers, keeps one copy of the step)
    if constexpr (TK == 128) {
      for (int i = 0; i < nsamp; i += kStages) {
        step128(i, StageC<0>{}, SampleC<true>{});
        step128(i + 1, StageC<1>{}, SampleC<true>{});
        step128(i + 2, StageC<2>{}, SampleC<true>{});
        step128(i + 3, StageC<3>{}, SampleC<true>{});
        step128(i + 4, StageC<4>{}, SampleC<true>{});
      }
    } else {
      for (int i = 0, st = 0; i < nsamp; ++i, st = st == kStages - 1 ? 0 : st + 1) step(i, st, SampleC<true>{});
    }
    __builtin_amdgcn_s_waitcnt(0x3F70);  // the requests past the sample tiles
    if (active) {
      const float s = sampled_start();
      if (l == 0) args.start[j] = s;
    }
    return;
  } else if constexpr (TK == 128) {
    for (int i = 0; i < ntiles; i += kStages) {
      step128(i, StageC<0>{}, SampleC<false>{});
      if (i + 1 >= ntiles) break;
      step128(i + 1, StageC<1>{}, SampleC<false>{});
      if (i + 2 >= ntiles) break;
      step128(i + 2, StageC<2>{}, SampleC<false>{});
      if (i + 3 >= ntiles) break;
      step128(i + 3, StageC<3>{}, SampleC<false>{});
      if (i + 4 >= ntiles) break;
      step128(i + 4, StageC<4>{}, SampleC<false>{});
    }
  } else if constexpr (DT == kFP8) {
    for (int i = 0; i < ntiles; i += kStages) {
      step(i, StageC<0>{}, SampleC<false>{});
      if (i + 1 >= ntiles) break;
      step(i + 1, StageC<1>{}, SampleC<false>{});
      if (i + 2 >= ntiles) break;
      step(i + 2, StageC<2>{}, SampleC<false>{});
      if (i + 3 >= ntiles) break;
      step(i + 3, StageC<3>{}, SampleC<false>{});
      if (i + 4 >= ntiles) break;
      step(i + 4, StageC<4>{}, SampleC<false>{});
    }
  } else {
    for (int i = 0, st = 0; i < ntiles; ++i, st = st == kStages - 1 ? 0 : st + 1) step(i, st, SampleC<false>{});
  }

  // the requests issued past the last tile: none may still be writing LDS
  // when the wave ends
  __builtin_amdgcn_s_waitcnt(0x3F70);
  if constexpr (kCertify) {
    // the check of a sampled start: a query that kept at least K entries (a
    // compaction keeps at least K) holds its whole top K; otherwise the
    // workgroup is flagged and its rows are streamed again, by the re-stream
    // launch, which writes the output instead.  A finite threshold means a
    // sampled start or a compaction, and after a compaction at least K are
    // kept, so the test needs no second read of the start.
    // The pre-pass cleared the workgroup's flag; a query that fails sets it
    // and writes nothing, the others write their rows (the re-stream writes
    // the same ones again).
    if (args.start != nullptr && !args.rerun_pass && active && thr > -__builtin_inff() && cnt + nst < args.K) {
      if (l == 0) args.rerun[blockIdx.x] = 1;
      return;
    }
  }
  if (!active) return;
  int32_t* const orow = args.out_idx + (int64_t)j * args.out_stride;
  float* const srow = args.out_score ? args.out_score + (int64_t)j * args.out_stride : nullptr;
  if constexpr (FULL) {
    wave_emit_row<32>(ckey, cidx, ncand_me, args.K, hist, orow, srow, [&](int c) __attribute__((always_inline)) {
      if constexpr (GATHER) return c < nbank ? bank[c] : anchor + 1 + (c - nbank);
      else return c;
    });
  } else {
    flush();
    wave_emit_topk<32>(ckey, cidx, cnt, args.K, hist, orow, srow);
  }
}

}  // namespace

bool dense_topk_supported(const ScanArgs& a) {
  // buffer offsets are 32-bit: the key rows up to the last query's position
  // (plus the tiles requested past it) must stay below 2 GiB
  const int64_t keys = a.pos0 + (a.nq - 1) * a.pos_stride + 1 + kAhead * 128;
  // bank refinement: every workgroup's 8 queries must sit in one group
  const bool shape_ok = a.bank == nullptr || (a.group % kWaves == 0 && a.nq % kWaves == 0 && a.pos_stride == 1);
  return shape_ok && a.H > 32 && a.H <= 64 && a.d == kD && keys * 2 * kD < (int64_t(1) << 31);
}

template <bool GATHER, bool FULL>
static void launch_dt(const ScanArgs& a, int dtype, dim3 grid, hipStream_t stream) {
  if (dtype == kBF16)
    hipLaunchKernelGGL((dense_topk_kernel<kBF16, GATHER, FULL, false>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((dense_topk_kernel<kFP8, GATHER, FULL, false>), grid, dim3(kThreads), 0, stream, a);
}

hipError_t launch_dense_topk(const ScanArgs& a, int dtype, hipStream_t stream) {
  const int64_t blocks = (a.nq + kWaves - 1) / kWaves;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  // full-row mode when every row's candidates fit its buffer (cap < 65536,
  // so the 16-bit histogram counters cannot overflow)
  const int64_t ncand_max =
      a.bank ? (int64_t)a.bank_stride + a.group - 1 : a.pos0 + (a.nq - 1) * a.pos_stride + 1;
  const bool full = ncand_max <= a.cap;
  if (a.bank) {
    if (full) launch_dt<true, true>(a, dtype, grid, stream);
    else launch_dt<true, false>(a, dtype, grid, stream);
  } else if (full) {
    launch_dt<false, true>(a, dtype, grid, stream);
  } else if (a.start != nullptr && ncand_max >= sample_min_row(dtype)) {
    // sampled start: the pre-pass, the stream, the re-stream of flagged
    // workgroups
    if (dtype == kBF16)
      hipLaunchKernelGGL((dense_topk_kernel<kBF16, false, false, true>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((dense_topk_kernel<kFP8, false, false, true>), grid, dim3(kThreads), 0, stream, a);
    launch_dt<false, false>(a, dtype, grid, stream);
    ScanArgs r = a;
    r.rerun_pass = 1;
    launch_dt<false, false>(r, dtype, grid, stream);
  } else {
    ScanArgs r = a;
    r.start = nullptr;  // no start: nothing to check
    launch_dt<false, false>(r, dtype, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace dsaidx
