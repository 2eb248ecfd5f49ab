// api.cpp -- the C ABI of libdsaidx.so (declared in include/dsa_indexer.h):
// host-side validation, workspace layout and kernel dispatch.  Every argument
// error is caught here, before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>
#include <algorithm>
#include <cmath>

#include "dsa_indexer.h"
#include "launch.h"

using namespace dsaidx;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return DSAIDX_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DSAIDX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxTopK = 2048;
constexpr int kMaxBank = 16384;
constexpr int kMaxHeads = 64;
// Rows per launch of the streaming kernel: bounds the candidate workspace.
constexpr int64_t kRowsPerLaunch = 16384;
constexpr int64_t kAnchorsPerLaunch = 4096;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Candidate-buffer entries per row: room for K survivors plus 2048 + K new
// arrivals between compactions (a multiple of 64, below 65536 for the 16-bit
// selection histograms).
int cap_for(int K) { return (2 * K + 2048 + 63) / 64 * 64; }

size_t cand_bytes_cap(int64_t rows, int cap) { return 2 * align_up((size_t)rows * (size_t)cap * 4u); }
size_t cand_bytes(int64_t rows, int K) { return cand_bytes_cap(rows, cap_for(K)); }
// the dense kernel's sampled start: a start per row and a flag per
// workgroup of 8 rows, after the candidate buffers
size_t sample_bytes(int64_t rows) { return align_up((size_t)rows * 4u) + align_up((size_t)(rows + 7) / 8 * 4u); }

// Group-bank rows whose candidates are bounded by the bank (refinement rows
// of at most P + G - 1 candidates, fallback rows before the first bank group)
// get a buffer that holds all of them: the dense kernel then keeps every
// score and a histogram instead of streaming the top K through compactions.
// The bound keeps a row's count in the 16-bit histogram counters (a multiple
// of 64 below 65536).  Dense prefill rows never get more than cap_for(K)
// entries, whatever their length.
constexpr int64_t kFullRowMax = 65472;
int full_cap(int K, int64_t ncand) {
  const int base = cap_for(K);
  if (ncand > kFullRowMax) return base;
  const int c = (int)((ncand + 63) / 64 * 64);
  return c > base ? c : base;
}

int row_bytes(int dtype, int d) { return dtype == DSAIDX_BF16 ? 2 * d : d; }

int check_shape(int dtype, int H, int d, int topk) {
  if (dtype != DSAIDX_BF16 && dtype != DSAIDX_FP8_E4M3)
    return fail(DSAIDX_ERR_INVALID_ARG, "dtype %d is not DSAIDX_BF16 or DSAIDX_FP8_E4M3", dtype);
  if (H < 1) return fail(DSAIDX_ERR_INVALID_ARG, "H = %d must be positive", H);
  if (H > kMaxHeads) return fail(DSAIDX_ERR_UNSUPPORTED, "H = %d above %d", H, kMaxHeads);
  if (d <= 0) return fail(DSAIDX_ERR_INVALID_ARG, "d = %d must be positive", d);
  const bool d_ok = dtype == DSAIDX_BF16 ? (d == 32 || d == 64 || d == 128) : (d == 64 || d == 128);
  if (!d_ok) return fail(DSAIDX_ERR_UNSUPPORTED, "d = %d unsupported for this dtype", d);
  if (topk < 1) return fail(DSAIDX_ERR_INVALID_ARG, "topk = %d must be positive", topk);
  if (topk > kMaxTopK) return fail(DSAIDX_ERR_UNSUPPORTED, "topk = %d above %d", topk, kMaxTopK);
  return DSAIDX_OK;
}

int check_prefill_common(const void* q, const float* q_scale, const void* k, const float* k_scale,
                         const float* w, int dtype, int64_t Tq, int64_t Tk, int H, int d,
                         int64_t q_pos0, int topk, const int32_t* out_idx, const float* out_score) {
  int rc = check_shape(dtype, H, d, topk);
  if (rc) return rc;
  if (Tq < 0 || Tk < 0 || q_pos0 < 0)
    return fail(DSAIDX_ERR_INVALID_ARG, "negative size (Tq=%lld Tk=%lld q_pos0=%lld)",
                (long long)Tq, (long long)Tk, (long long)q_pos0);
  if (q_pos0 + Tq > Tk)
    return fail(DSAIDX_ERR_INVALID_ARG, "q_pos0 + Tq = %lld exceeds Tk = %lld",
                (long long)(q_pos0 + Tq), (long long)Tk);
  if (Tk > INT32_MAX) return fail(DSAIDX_ERR_UNSUPPORTED, "Tk above INT32_MAX");
  if (Tq > 0 && (!q || !k || !w || !out_idx))
    return fail(DSAIDX_ERR_INVALID_ARG, "null q, k, w or out_idx");
  const bool fp8 = dtype == DSAIDX_FP8_E4M3;
  if (Tq > 0 && fp8 && (!q_scale || !k_scale))
    return fail(DSAIDX_ERR_INVALID_ARG, "fp8 inputs need q_scale and k_scale");
  if (!fp8 && (q_scale || k_scale))
    return fail(DSAIDX_ERR_INVALID_ARG, "bf16 inputs take no scales (pass NULL)");
  if (!aligned16(q) || !aligned16(k) || !aligned16(w) || !aligned16(out_idx) ||
      !aligned16(out_score))
    return fail(DSAIDX_ERR_INVALID_ARG, "q, k, w and outputs must be 16-byte aligned");
  if (((uintptr_t)q_scale & 3u) || ((uintptr_t)k_scale & 3u))
    return fail(DSAIDX_ERR_INVALID_ARG, "scales must be 4-byte aligned");
  return DSAIDX_OK;
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return DSAIDX_OK;
  if (!ws) return fail(DSAIDX_ERR_WORKSPACE, "null workspace (%zu bytes needed)", need);
  if (!aligned16(ws)) return fail(DSAIDX_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (ws_bytes < need)
    return fail(DSAIDX_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  return DSAIDX_OK;
}

// The environment variable DSAIDX_SAMPLE_RERUN=1 makes the dense kernel's
// sampled start fail on purpose, so that the rows it covers are
// streamed a second time from -inf: a test of that path (results unchanged).
static int sample_test_forced() {
  const char* v = std::getenv("DSAIDX_SAMPLE_RERUN");
  return v != nullptr && v[0] == '1';
}

// Dense rows [r0, r1) of a prefill-shaped call, sliced into launches of at
// most kRowsPerLaunch rows.  Rows whose candidates all fit a buffer of `cap`
// entries (position + 1 <= cap) get launches of their own, so the dense
// kernel keeps their whole (short) rows; longer rows stream their top K
// through the same buffers.  `sample`: the workspace also holds
// sample_bytes(rows) after the candidate buffers of `rows` rows (rows >= every
// launch's n), so that long rows can stream from a sampled start.
hipError_t run_dense(const void* q, const float* q_scale, const void* k, const float* k_scale,
                     const float* w, int dtype, int H, int d, int64_t q_pos0, int64_t r0,
                     int64_t r1, int topk, int cap, int32_t* out_idx, float* out_score, void* ws,
                     hipStream_t stream, bool sample = false) {
  const int rb = row_bytes(dtype, d);
  int64_t split = (int64_t)cap - q_pos0;  // first row with more than cap candidates
  split = split < r0 ? r0 : (split > r1 ? r1 : split);
  for (int64_t s = r0; s < r1;) {
    const int64_t end = s < split ? split : r1;
    const int64_t n = end - s < kRowsPerLaunch ? end - s : kRowsPerLaunch;
    ScanArgs a{};
    a.q = (const uint8_t*)q + s * H * (int64_t)rb;
    a.q_scale = q_scale ? q_scale + s : nullptr;
    a.w = w + s * H;
    a.k = k;
    a.k_scale = k_scale;
    a.H = H;
    a.d = d;
    a.nq = n;
    a.pos0 = q_pos0 + s;
    a.pos_stride = 1;
    a.bank = nullptr;
    a.K = topk;
    a.cap = cap;
    a.cand_key = (uint32_t*)ws;
    a.cand_idx = (int32_t*)((uint8_t*)ws + align_up((size_t)n * cap * 4u));
    a.out_idx = out_idx + s * topk;
    a.out_score = out_score ? out_score + s * topk : nullptr;
    a.out_stride = topk;
    if (sample) {
      const int64_t rows = r1 - r0 < kRowsPerLaunch ? r1 - r0 : kRowsPerLaunch;
      uint8_t* sws = (uint8_t*)ws + cand_bytes_cap(rows, cap);
      a.start = (float*)sws;
      a.rerun = (int32_t*)(sws + align_up((size_t)rows * 4u));
      a.sample_test = sample_test_forced();
    }
    hipError_t e = launch_scan_topk(a, dtype, stream);
    if (e != hipSuccess) return e;
    s += n;
  }
  return hipSuccess;
}

struct GroupPlan {
  int64_t NG, nfull, g0;  // groups; complete groups; first bank group
};

GroupPlan plan_groups(int64_t Tq, int64_t q_pos0, int G, int P, unsigned flags) {
  GroupPlan p;
  p.NG = (Tq + G - 1) / G;
  p.nfull = Tq / G;
  if (flags & DSAIDX_FORCE_BANK) {
    p.g0 = 0;
  } else {
    // smallest g with anchor q_pos0 + gG seeing more than P keys
    const int64_t need = (int64_t)P - q_pos0;  // gG >= need  <=>  anchor + 1 > P
    p.g0 = need <= 0 ? 0 : (need + G - 1) / G;
  }
  if (p.g0 > p.nfull) p.g0 = p.nfull;
  return p;
}

// The pooled group query and gates of the bank groups (DSAIDX_POOL_MEAN).
size_t pool_q_bytes(int64_t nelig, int H, int d) {
  return align_up((size_t)(nelig > 0 ? nelig : 0) * H * d * 2u);
}
size_t pool_w_bytes(int64_t nelig, int H) {
  return align_up((size_t)(nelig > 0 ? nelig : 0) * H * 4u);
}

// workspace: [bank groups' banks, when out_bank is NULL] [pooled group query
// and gates, with DSAIDX_POOL_MEAN] [candidate buffers of one launch]
size_t group_ws_bytes(int64_t Tq, int H, int d, int G, int P, int topk, unsigned flags,
                      int64_t q_pos0, bool bank_in_ws) {
  const GroupPlan p = plan_groups(Tq, q_pos0, G, P, flags);
  const int64_t nelig = p.nfull - p.g0;
  size_t bank = bank_in_ws ? align_up((size_t)(nelig > 0 ? nelig : 0) * P * 4u) : 0;
  if (flags & DSAIDX_POOL_MEAN) bank += pool_q_bytes(nelig, H, d) + pool_w_bytes(nelig, H);
  const int64_t anchors = nelig < kAnchorsPerLaunch ? nelig : kAnchorsPerLaunch;
  const int64_t rows = Tq < kRowsPerLaunch ? Tq : kRowsPerLaunch;
  // the group scan's candidate buffers and its sampled starts
  size_t scan = anchors > 0 ? cand_bytes(anchors, P) + sample_bytes(anchors) : 0;
  size_t refine = rows > 0 ? cand_bytes_cap(rows, full_cap(topk, (int64_t)P + G - 1)) : 0;
  return bank + (scan > refine ? scan : refine);
}

}  // namespace

namespace dsaidx {
// The calling thread's error message, for entry points defined in other files.
int report_error(int code, const char* msg) { return fail(code, "%s", msg); }
int report_hip_error(hipError_t e, const char* what) { return hip_fail(e, what); }
}  // namespace dsaidx

extern "C" {

const char* indexer_last_error(void) { return g_last_error.c_str(); }

size_t indexer_prefill_workspace_size(int64_t Tq, int64_t Tk, int H, int d, int topk, int dtype) {
  (void)Tk; (void)H; (void)d; (void)dtype;
  if (Tq <= 0 || topk <= 0) return 0;
  const int64_t rows = Tq < kRowsPerLaunch ? Tq : kRowsPerLaunch;
  return cand_bytes(rows, topk) + sample_bytes(rows);
}

int indexer_prefill(const void* q, const float* q_scale, const void* k, const float* k_scale,
                    const float* w, int dtype, int64_t Tq, int64_t Tk, int H, int d,
                    int64_t q_pos0, int topk, int32_t* out_idx, float* out_score, void* ws,
                    size_t ws_bytes, void* stream) {
  int rc = check_prefill_common(q, q_scale, k, k_scale, w, dtype, Tq, Tk, H, d, q_pos0, topk,
                                out_idx, out_score);
  if (rc) return rc;
  rc = check_ws(ws, ws_bytes, indexer_prefill_workspace_size(Tq, Tk, H, d, topk, dtype));
  if (rc) return rc;
  if (Tq == 0) return ok();
  hipError_t e = run_dense(q, q_scale, k, k_scale, w, dtype, H, d, q_pos0, 0, Tq, topk,
                           cap_for(topk), out_idx, out_score, ws, (hipStream_t)stream, true);
  if (e != hipSuccess) return hip_fail(e, "indexer_prefill launch");
  return ok();
}

// decode workspace: histograms [B, bins] + candidate counts [B] | row
// emission state [B, 4] | candidate keys and indices [B, cap] each | per-span
// counts [B, nblk]: list entries, entries above b*, output offsets | compact
// lists [B, nblk, kpb] of indices and of scores
struct DecodeWs {
  size_t hist, rowsel, ckey, cidx, clcnt, above, off, clidx, clsc, total;
};

// keys per scan workgroup: about 512 workgroups per call (two per CU), a
// multiple of 256 keys and at most what one workgroup's LDS score stages
// hold; R rows per scan workgroup (they share its keys)
static int64_t decode_keys_per_block(int B, int64_t Nmax, int R = 1) {
  const int64_t target = ((int64_t)(B / R) * Nmax + 511) / 512;
  int64_t kpb = (target + 255) / 256 * 256;
  const int64_t row = (Nmax + 255) / 256 * 256;
  if (kpb > row) kpb = row;
  if (kpb > dec_max_kpb(R)) kpb = dec_max_kpb(R);
  return kpb < 256 ? 256 : kpb;
}

static DecodeWs decode_ws(int B, int64_t Nmax, int R = 1) {
  const size_t kpb = (size_t)decode_keys_per_block(B, Nmax, R);
  const size_t nblk = ((size_t)Nmax + kpb - 1) / kpb;
  DecodeWs w{};
  w.hist = 0;
  w.rowsel = w.hist + align_up(((size_t)B * kDecHistBins + (size_t)B) * 4u);
  w.ckey = w.rowsel + align_up((size_t)B * 16u);
  w.cidx = w.ckey + align_up((size_t)B * kDecCandCap * 4u);
  w.clcnt = w.cidx + align_up((size_t)B * kDecCandCap * 4u);
  w.above = w.clcnt + align_up((size_t)B * nblk * kDecListSegs * 4u);
  w.off = w.above + align_up((size_t)B * nblk * 4u);
  w.clidx = w.off + align_up((size_t)B * nblk * 4u);
  w.clsc = w.clidx + align_up((size_t)B * nblk * kpb * 4u);
  w.total = w.clsc + align_up((size_t)B * nblk * kpb * 4u);
  return w;
}

// The decode pipeline's arguments over `rows` rows of at most Nmax keys, its
// workspace at ws (decode_ws(rows, Nmax, R).total bytes), R rows per scan
// workgroup.
static DecodeArgs decode_args(const void* q, const float* w, const int32_t* lens, int rows,
                              int64_t Nmax, int H, int d, int K, void* ws, int32_t* out_idx,
                              float* out_score, int R = 1) {
  DecodeArgs a{};
  a.q = q;
  a.w = w;
  a.seq_lens = lens;
  a.B = rows;
  a.H = H;
  a.d = d;
  a.Nmax = Nmax;
  a.K = K;
  a.scan_rows = R;
  const DecodeWs lay = decode_ws(rows, Nmax, R);
  uint8_t* base = (uint8_t*)ws;
  a.kpb = decode_keys_per_block(rows, Nmax, R);
  a.nblk = (int)((Nmax + a.kpb - 1) / a.kpb);
  a.hist = (uint32_t*)(base + lay.hist);
  a.cand_cnt = (int32_t*)(a.hist + (size_t)rows * kDecHistBins);
  a.rowsel = (uint32_t*)(base + lay.rowsel);
  a.cand_key = (uint32_t*)(base + lay.ckey);
  a.cand_idx = (int32_t*)(base + lay.cidx);
  a.span_above = (int32_t*)(base + lay.above);
  a.span_off = (int32_t*)(base + lay.off);
  a.cl_cnt = (int32_t*)(base + lay.clcnt);
  a.cl_idx = (int32_t*)(base + lay.clidx);
  a.cl_sc = (float*)(base + lay.clsc);
  a.out_idx = out_idx;
  a.out_score = out_score;
  return a;
}

size_t indexer_decode_workspace_size(int B, int64_t Nmax, int H, int d, int topk) {
  (void)H; (void)d; (void)topk;
  if (B <= 0 || Nmax <= 0) return 0;
  return decode_ws(B, Nmax).total;
}

int indexer_decode(const void* q, const uint8_t* k_cache, const float* k_scale, const float* w,
                   const int32_t* seq_lens, int B, int64_t Nmax, int H, int d, int topk,
                   int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(DSAIDX_FP8_E4M3, H, d, topk);
  if (rc) return rc;
  if (B < 0 || Nmax < 0)
    return fail(DSAIDX_ERR_INVALID_ARG, "negative size (B=%d Nmax=%lld)", B, (long long)Nmax);
  if (Nmax > INT32_MAX) return fail(DSAIDX_ERR_UNSUPPORTED, "Nmax above INT32_MAX");
  if (B > 0 && (!q || !k_cache || !k_scale || !w || !seq_lens || !out_idx))
    return fail(DSAIDX_ERR_INVALID_ARG, "null q, k_cache, k_scale, w, seq_lens or out_idx");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(w) || !aligned16(out_idx) ||
      !aligned16(out_score))
    return fail(DSAIDX_ERR_INVALID_ARG, "q, k_cache, w and outputs must be 16-byte aligned");
  if (((uintptr_t)k_scale & 3u) || ((uintptr_t)seq_lens & 3u))
    return fail(DSAIDX_ERR_INVALID_ARG, "k_scale and seq_lens must be 4-byte aligned");
  rc = check_ws(ws, ws_bytes, indexer_decode_workspace_size(B, Nmax, H, d, topk));
  if (rc) return rc;
  if (B == 0) return ok();
  DecodeArgs a = decode_args(q, w, seq_lens, B, Nmax, H, d, topk, ws, out_idx, out_score);
  a.kc = k_cache;
  a.k_scale = k_scale;
  hipError_t e = launch_decode(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "indexer_decode launch");
  return ok();
}

int64_t indexer_group_bank_pairs(int64_t Tq, int64_t q_pos0, int G, int P, unsigned flags) {
  if (Tq < 0 || q_pos0 < 0 || G <= 0 || P <= 0) return -1;
  const GroupPlan p = plan_groups(Tq, q_pos0, G, P, flags);
  int64_t pairs = 0;
  // original indexer rows: [0, g0*G) and [nfull*G, Tq); row i scores q_pos0+i+1 keys
  auto tri = [&](int64_t r0, int64_t r1) {
    for (int64_t i = r0; i < r1; ++i) pairs += q_pos0 + i + 1;
  };
  tri(0, p.g0 * G);
  tri(p.nfull * G, Tq);
  for (int64_t g = p.g0; g < p.nfull; ++g) {
    const int64_t anchor = q_pos0 + g * G;
    const int64_t nb = anchor + 1 < P ? anchor + 1 : P;
    pairs += anchor + 1 + (int64_t)G * nb + (int64_t)G * (G - 1) / 2;
  }
  return pairs;
}

size_t indexer_group_bank_workspace_size(int64_t Tq, int64_t Tk, int H, int Hs, int d, int G,
                                         int P, int topk, int dtype, unsigned flags) {
  (void)Tk; (void)Hs; (void)dtype;
  if (Tq <= 0 || G <= 0 || P <= 0 || topk <= 0 || H <= 0 || d <= 0) return 0;
  // sized for the worst case: a bank for every complete group, kept in ws
  return group_ws_bytes(Tq, H, d, G, P, topk, DSAIDX_FORCE_BANK | (flags & DSAIDX_POOL_MEAN), 0,
                        true);
}

}  // extern "C"

namespace {

// Argument checks of a group-bank call (everything but the workspace).
int check_group_bank(const void* q, const float* q_scale, const void* k, const float* k_scale,
                     const float* w, int dtype, int64_t Tq, int64_t Tk, int H, int d,
                     int64_t q_pos0, const void* qbar, const float* qbar_scale,
                     const float* wbar, int Hs, int G, int P, int topk, unsigned flags,
                     const int32_t* out_idx, const int32_t* out_bank, const float* out_score) {
  int rc = check_prefill_common(q, q_scale, k, k_scale, w, dtype, Tq, Tk, H, d, q_pos0, topk,
                                out_idx, out_score);
  if (rc) return rc;
  if (G != 4 && G != 8 && G != 16)
    return fail(DSAIDX_ERR_UNSUPPORTED, "group size G = %d not in {4, 8, 16}", G);
  if (P < topk) return fail(DSAIDX_ERR_INVALID_ARG, "bank size P = %d below topk = %d", P, topk);
  if (P > kMaxBank) return fail(DSAIDX_ERR_UNSUPPORTED, "bank size P = %d above %d", P, kMaxBank);
  if (Hs < 1) return fail(DSAIDX_ERR_INVALID_ARG, "Hs = %d must be positive", Hs);
  if (Hs > kMaxHeads) return fail(DSAIDX_ERR_UNSUPPORTED, "Hs = %d above %d", Hs, kMaxHeads);
  if (q_pos0 % G) return fail(DSAIDX_ERR_INVALID_ARG, "q_pos0 must be a multiple of G");
  if (flags & ~(unsigned)(DSAIDX_FORCE_BANK | DSAIDX_POOL_MEAN))
    return fail(DSAIDX_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  const bool fp8 = dtype == DSAIDX_FP8_E4M3;
  const bool pool = (flags & DSAIDX_POOL_MEAN) != 0;
  if (pool) {
    if (fp8) return fail(DSAIDX_ERR_UNSUPPORTED, "DSAIDX_POOL_MEAN takes bf16 queries");
    if (qbar || wbar || qbar_scale)
      return fail(DSAIDX_ERR_INVALID_ARG, "DSAIDX_POOL_MEAN takes NULL qbar, wbar and qbar_scale");
    if (Hs != H) return fail(DSAIDX_ERR_INVALID_ARG, "DSAIDX_POOL_MEAN needs Hs == H");
  }
  if (Tq > 0 && !pool && (!qbar || !wbar)) return fail(DSAIDX_ERR_INVALID_ARG, "null qbar or wbar");
  if (Tq > 0 && fp8 && !qbar_scale)
    return fail(DSAIDX_ERR_INVALID_ARG, "fp8 inputs need qbar_scale");
  if (!fp8 && qbar_scale) return fail(DSAIDX_ERR_INVALID_ARG, "bf16 qbar takes no scale");
  if (!aligned16(qbar) || !aligned16(wbar) || !aligned16(out_bank))
    return fail(DSAIDX_ERR_INVALID_ARG, "qbar, wbar and out_bank must be 16-byte aligned");
  if ((uintptr_t)qbar_scale & 3u) return fail(DSAIDX_ERR_INVALID_ARG, "qbar_scale misaligned");
  return DSAIDX_OK;
}

// Enqueue a checked group-bank call (Tq > 0, workspace large enough).
int run_group_bank(const void* q, const float* q_scale, const void* k, const float* k_scale,
                   const float* w, int dtype, int64_t Tq, int H, int d, int64_t q_pos0,
                   const void* qbar, const float* qbar_scale, const float* wbar, int Hs, int G,
                   int P, int topk, unsigned flags, int32_t* out_idx, int32_t* out_bank,
                   float* out_score, void* ws, hipStream_t st) {
  const bool pool = (flags & DSAIDX_POOL_MEAN) != 0;
  const GroupPlan p = plan_groups(Tq, q_pos0, G, P, flags);
  const int64_t nelig = p.nfull - p.g0;
  const int rb = row_bytes(dtype, d);
  int32_t* bank;
  void* cand_ws;
  if (out_bank) {
    bank = out_bank + p.g0 * (int64_t)P;
    cand_ws = ws;
    hipError_t e = launch_fill_i32(out_bank, p.g0 * (int64_t)P, -1, st);
    if (e == hipSuccess)
      e = launch_fill_i32(out_bank + p.nfull * (int64_t)P, (p.NG - p.nfull) * (int64_t)P, -1, st);
    if (e != hipSuccess) return hip_fail(e, "indexer_group_bank bank fill");
  } else {
    bank = (int32_t*)ws;
    cand_ws = (uint8_t*)ws + align_up((size_t)(nelig > 0 ? nelig : 0) * P * 4u);
  }
  // the bank groups' group query: the caller's, or the mean of each group's
  // own queries and gates (pooled groups g0 .. nfull-1, rows from 0)
  const void* gq = qbar;
  const float* gw = wbar;
  int64_t gq_row0 = 0;  // row of qbar / wbar holding group g0
  if (pool) {
    PoolArgs pa{};
    pa.q = q;
    pa.w = w;
    pa.H = H;
    pa.d = d;
    pa.G = G;
    pa.g0 = p.g0;
    pa.ngroups = nelig > 0 ? nelig : 0;
    pa.qbar = cand_ws;
    pa.wbar = (float*)((uint8_t*)cand_ws + pool_q_bytes(nelig, H, d));
    gq = pa.qbar;
    gw = pa.wbar;
    gq_row0 = -p.g0;
    cand_ws = (uint8_t*)cand_ws + pool_q_bytes(nelig, H, d) + pool_w_bytes(nelig, H);
    hipError_t e = launch_pool_mean(pa, st);
    if (e != hipSuccess) return hip_fail(e, "indexer_group_bank pooling launch");
  }

  // 1. original indexer for the rows whose groups build no bank; those before
  // the first bank group see at most P + G - 1 keys, so their rows fit the
  // full-row buffers the workspace holds for the refinement
  hipError_t e = run_dense(q, q_scale, k, k_scale, w, dtype, H, d, q_pos0, 0, p.g0 * G, topk,
                           full_cap(topk, q_pos0 + p.g0 * G), out_idx, out_score, cand_ws, st);
  if (e == hipSuccess)
    e = run_dense(q, q_scale, k, k_scale, w, dtype, H, d, q_pos0, p.nfull * G, Tq, topk, cap_for(topk),
                  out_idx, out_score, cand_ws, st);
  if (e != hipSuccess) return hip_fail(e, "indexer_group_bank fallback launch");

  // 2. group scan: each bank group's anchor scores its prefix with the group
  //    indexer and keeps the top P (Eq. (8), (13))
  const int capP = cap_for(P);
  for (int64_t s = 0; s < nelig; s += kAnchorsPerLaunch) {
    const int64_t n = nelig - s < kAnchorsPerLaunch ? nelig - s : kAnchorsPerLaunch;
    const int64_t g = p.g0 + s;
    ScanArgs a{};
    a.q = (const uint8_t*)gq + (g + gq_row0) * Hs * (int64_t)rb;
    a.q_scale = qbar_scale ? qbar_scale + g : nullptr;
    a.w = gw + (g + gq_row0) * Hs;
    a.k = k;
    a.k_scale = k_scale;
    a.H = Hs;
    a.d = d;
    a.nq = n;
    a.pos0 = q_pos0 + g * G;
    a.pos_stride = G;
    a.bank = nullptr;
    a.K = P;
    a.cap = capP;
    a.cand_key = (uint32_t*)cand_ws;
    a.cand_idx = (int32_t*)((uint8_t*)cand_ws + align_up((size_t)n * capP * 4u));
    a.out_idx = bank + s * (int64_t)P;
    a.out_score = nullptr;
    a.out_stride = P;
    // long anchor rows stream from a sampled start (the dense kernel only)
    const int64_t anchors = nelig < kAnchorsPerLaunch ? nelig : kAnchorsPerLaunch;
    uint8_t* sws = (uint8_t*)cand_ws + cand_bytes(anchors, P);
    a.start = (float*)sws;
    a.rerun = (int32_t*)(sws + align_up((size_t)anchors * 4u));
    a.sample_test = sample_test_forced();
    e = launch_scan_topk(a, dtype, st);
    if (e != hipSuccess) return hip_fail(e, "indexer_group_bank group scan launch");
  }

  // 3. refinement: every member of a bank group scores bank U {t+1..i} with the
  //    original indexer and keeps its top K (Eq. (14))
  const int cap = full_cap(topk, (int64_t)P + G - 1);  // every refinement row fits its buffer
  const int64_t groups_per_launch = kRowsPerLaunch / G;
  for (int64_t s = 0; s < nelig; s += groups_per_launch) {
    const int64_t ng = nelig - s < groups_per_launch ? nelig - s : groups_per_launch;
    const int64_t r0 = (p.g0 + s) * G;  // first row of the launch
    const int64_t n = ng * G;
    ScanArgs a{};
    a.q = (const uint8_t*)q + r0 * H * (int64_t)rb;
    a.q_scale = q_scale ? q_scale + r0 : nullptr;
    a.w = w + r0 * H;
    a.k = k;
    a.k_scale = k_scale;
    a.H = H;
    a.d = d;
    a.nq = n;
    a.pos0 = q_pos0 + r0;
    a.pos_stride = 1;
    a.bank = bank + s * (int64_t)P;
    a.bank_stride = P;
    a.group = G;
    a.K = topk;
    a.cap = cap;
    a.cand_key = (uint32_t*)cand_ws;
    a.cand_idx = (int32_t*)((uint8_t*)cand_ws + align_up((size_t)n * cap * 4u));
    a.out_idx = out_idx + r0 * topk;
    a.out_score = out_score ? out_score + r0 * topk : nullptr;
    a.out_stride = topk;
    e = launch_scan_topk(a, dtype, st);
    if (e != hipSuccess) return hip_fail(e, "indexer_group_bank refine launch");
  }
  return DSAIDX_OK;
}

}  // namespace

extern "C" {

int indexer_group_bank(const void* q, const float* q_scale, const void* k, const float* k_scale,
                       const float* w, int dtype, int64_t Tq, int64_t Tk, int H, int d,
                       int64_t q_pos0, const void* qbar, const float* qbar_scale,
                       const float* wbar, int Hs, int G, int P, int topk, unsigned flags,
                       int32_t* out_idx, int32_t* out_bank, float* out_score, void* ws,
                       size_t ws_bytes, void* stream) {
  int rc = check_group_bank(q, q_scale, k, k_scale, w, dtype, Tq, Tk, H, d, q_pos0, qbar, qbar_scale,
                            wbar, Hs, G, P, topk, flags, out_idx, out_bank, out_score);
  if (rc) return rc;
  rc = check_ws(ws, ws_bytes,
                group_ws_bytes(Tq, H, d, G, P, topk, flags, q_pos0, out_bank == nullptr));
  if (rc) return rc;
  if (Tq == 0) return ok();
  rc = run_group_bank(q, q_scale, k, k_scale, w, dtype, Tq, H, d, q_pos0, qbar, qbar_scale, wbar, Hs, G,
                      P, topk, flags, out_idx, out_bank, out_score, ws, (hipStream_t)stream);
  return rc ? rc : ok();
}

// ------------------------------------------------------ layer-wise dispatch

size_t indexer_layers_workspace_size(const dsaidx_layer* layers, int nlayers, int64_t Tq, int64_t Tk,
                                     int H, int d, int topk, int dtype) {
  if (!layers || nlayers <= 0 || Tq <= 0 || topk <= 0 || H <= 0 || d <= 0) return 0;
  size_t need = 0;
  for (int i = 0; i < nlayers; ++i) {
    const dsaidx_layer& L = layers[i];
    size_t n;
    if (L.G == 0) {
      n = indexer_prefill_workspace_size(Tq, Tk, H, d, topk, dtype);
    } else {
      if (L.G < 0 || L.P <= 0) return 0;
      // any q_pos0: as many banks as complete groups, kept in ws without out_bank
      n = group_ws_bytes(Tq, H, d, L.G, L.P, topk, DSAIDX_FORCE_BANK | (L.flags & DSAIDX_POOL_MEAN), 0,
                         L.out_bank == nullptr);
    }
    if (n > need) need = n;
  }
  return need;
}

int indexer_layers(const dsaidx_layer* layers, int nlayers, int dtype, int64_t Tq, int64_t Tk, int H,
                   int d, int64_t q_pos0, int topk, void* ws, size_t ws_bytes, void* stream) {
  if (nlayers < 0) return fail(DSAIDX_ERR_INVALID_ARG, "nlayers = %d is negative", nlayers);
  if (nlayers > 0 && !layers) return fail(DSAIDX_ERR_INVALID_ARG, "null layers");
  // every layer is checked before anything is enqueued
  size_t need = 0;
  for (int i = 0; i < nlayers; ++i) {
    const dsaidx_layer& L = layers[i];
    int rc;
    size_t n;
    if (L.G == 0) {
      if (L.qbar || L.qbar_scale || L.wbar || L.out_bank || L.flags)
        return fail(DSAIDX_ERR_INVALID_ARG, "layer %d: an original-indexer layer (G = 0) takes no group "
                    "query, bank or flags", i);
      rc = check_prefill_common(L.q, L.q_scale, L.k, L.k_scale, L.w, dtype, Tq, Tk, H, d, q_pos0, topk,
                                L.out_idx, L.out_score);
      n = indexer_prefill_workspace_size(Tq, Tk, H, d, topk, dtype);
    } else {
      rc = check_group_bank(L.q, L.q_scale, L.k, L.k_scale, L.w, dtype, Tq, Tk, H, d, q_pos0, L.qbar,
                            L.qbar_scale, L.wbar, L.Hs, L.G, L.P, topk, L.flags, L.out_idx, L.out_bank,
                            L.out_score);
      n = rc ? 0 : group_ws_bytes(Tq, H, d, L.G, L.P, topk, L.flags, q_pos0, L.out_bank == nullptr);
    }
    if (rc) {
      const std::string msg = g_last_error;
      return fail(rc, "layer %d: %s", i, msg.c_str());
    }
    if (n > need) need = n;
  }
  int rc = check_ws(ws, ws_bytes, need);
  if (rc) return rc;
  if (Tq == 0) return ok();
  hipStream_t st = (hipStream_t)stream;
  for (int i = 0; i < nlayers; ++i) {
    const dsaidx_layer& L = layers[i];
    if (L.G == 0) {
      hipError_t e = run_dense(L.q, L.q_scale, L.k, L.k_scale, L.w, dtype, H, d, q_pos0, 0, Tq, topk,
                               cap_for(topk), L.out_idx, L.out_score, ws, st, true);
      if (e != hipSuccess) return hip_fail(e, "indexer_layers launch");
    } else {
      rc = run_group_bank(L.q, L.q_scale, L.k, L.k_scale, L.w, dtype, Tq, H, d, q_pos0, L.qbar, L.qbar_scale,
                          L.wbar, L.Hs, L.G, L.P, topk, L.flags, L.out_idx, L.out_bank, L.out_score, ws, st);
      if (rc) return rc;
    }
  }
  return ok();
}

// ---------------------------------------------------------------- MTP

// workspace: anchor rows' key sources and lengths | refinement rows' | banks
// (when out_bank is NULL) | pooled group queries and gates (DSAIDX_POOL_MEAN) |
// gathered candidate keys and scales | the decode pipeline's workspace (the
// anchor scan and the refinement run one after the other and share it)
struct MtpWs {
  size_t a_kc, a_ks, a_len, r_kc, r_ks, r_len, r_len2, bank, pq, pw, gk, gs, dec, total;
};

// anchor rows per scan workgroup: all the anchors of a window (up to 4) read
// the same cache, so one pass over it serves them when their heads fit
static int mtp_anchor_rows(int B, int m, int Hs, int G) {
  const int ngs = m / G;
  for (int R : {4, 2})
    if (ngs % R == 0 && dec_scan_rows_ok(R, Hs, B * ngs)) return R;
  return 1;
}

static MtpWs mtp_ws(int B, int64_t Nmax, int m, int H, int Hs, int d, int G, int P, unsigned flags,
                    bool bank_in_ws) {
  const size_t na = (size_t)B * (m / G), nr = (size_t)B * m, cand = (size_t)P + G - 1;
  MtpWs w{};
  w.a_kc = 0;
  w.a_ks = w.a_kc + align_up(na * 8u);
  w.a_len = w.a_ks + align_up(na * 8u);
  w.r_kc = w.a_len + align_up(na * 4u);
  w.r_ks = w.r_kc + align_up(nr * 8u);
  w.r_len = w.r_ks + align_up(nr * 8u);
  w.r_len2 = w.r_len + align_up(nr * 4u);
  w.bank = w.r_len2 + align_up(nr * 4u);
  w.pq = w.bank + (bank_in_ws ? align_up(na * P * 4u) : 0);
  const bool pool = (flags & DSAIDX_POOL_MEAN) != 0;
  w.pw = w.pq + (pool ? align_up(na * H * d * 2u) : 0);
  w.gk = w.pw + (pool ? align_up(na * H * 4u) : 0);
  w.gs = w.gk + align_up(na * cand * d);
  w.dec = w.gs + align_up(na * cand * 4u);
  size_t dw = decode_ws((int)na, Nmax, mtp_anchor_rows(B, m, Hs, G)).total;
  const size_t dr = decode_ws((int)nr, Nmax).total, db = decode_ws((int)nr, (int64_t)cand).total;
  if (dr > dw) dw = dr;
  if (db > dw) dw = db;
  w.total = w.dec + dw;
  return w;
}

size_t indexer_mtp_workspace_size(int B, int64_t Nmax, int m, int H, int Hs, int d, int G, int P,
                                  int topk, unsigned flags) {
  (void)topk;
  if (B <= 0 || Nmax <= 0 || m <= 0 || G <= 0 || m % G || P <= 0 || H <= 0 || d <= 0) return 0;
  return mtp_ws(B, Nmax, m, H, Hs, d, G, P, flags, true).total;
}

int64_t indexer_mtp_pairs(const int32_t* prefix_lens, int B, int64_t Nmax, int m, int G, int P,
                          unsigned flags) {
  if (B < 0 || m <= 0 || G <= 0 || m % G || P <= 0 || Nmax < m || (B > 0 && !prefix_lens))
    return -1;
  int64_t pairs = 0;
  for (int b = 0; b < B; ++b) {
    int64_t N = prefix_lens[b];
    N = N < 1 ? 1 : (N > Nmax - m + 1 ? Nmax - m + 1 : N);  // as the device clamps it
    if (N <= P || (flags & DSAIDX_NO_BANK)) {
      pairs += m * N + (int64_t)m * (m - 1) / 2;  // every query: N + r keys
      continue;
    }
    for (int g = 0; g < m / G; ++g)
      pairs += N + (int64_t)g * G + (int64_t)G * P + (int64_t)G * (G - 1) / 2;
  }
  return pairs;
}

int indexer_mtp(const void* q, const uint8_t* k_cache, const float* k_scale, const float* w,
                const void* qbar, const float* wbar, const int32_t* prefix_lens, int B,
                int64_t Nmax, int m, int H, int Hs, int d, int G, int P, int topk, unsigned flags,
                int32_t* out_idx, int32_t* out_bank, float* out_score, void* ws, size_t ws_bytes,
                void* stream) {
  int rc = check_shape(DSAIDX_FP8_E4M3, H, d, topk);
  if (rc) return rc;
  if (B < 0 || Nmax < 0 || m < 1)
    return fail(DSAIDX_ERR_INVALID_ARG, "bad size (B=%d Nmax=%lld m=%d)", B, (long long)Nmax, m);
  if (G != 4 && G != 8 && G != 16)
    return fail(DSAIDX_ERR_UNSUPPORTED, "group size G = %d not in {4, 8, 16}", G);
  if (m % G) return fail(DSAIDX_ERR_INVALID_ARG, "window m = %d is not a multiple of G = %d", m, G);
  if (m > 64) return fail(DSAIDX_ERR_UNSUPPORTED, "window m = %d above 64", m);
  if (Nmax < m) return fail(DSAIDX_ERR_INVALID_ARG, "Nmax = %lld below the window m", (long long)Nmax);
  if (Nmax > INT32_MAX) return fail(DSAIDX_ERR_UNSUPPORTED, "Nmax above INT32_MAX");
  if ((int64_t)B * m > 65535) return fail(DSAIDX_ERR_UNSUPPORTED, "B * m above 65535");
  if (P < topk) return fail(DSAIDX_ERR_INVALID_ARG, "bank size P = %d below topk = %d", P, topk);
  if (P > kMaxBank) return fail(DSAIDX_ERR_UNSUPPORTED, "bank size P = %d above %d", P, kMaxBank);
  if (flags & ~(unsigned)(DSAIDX_POOL_MEAN | DSAIDX_NO_BANK))
    return fail(DSAIDX_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  const bool pool = (flags & DSAIDX_POOL_MEAN) != 0;
  const bool no_bank = (flags & DSAIDX_NO_BANK) != 0;
  if (pool && no_bank)
    return fail(DSAIDX_ERR_INVALID_ARG, "DSAIDX_POOL_MEAN and DSAIDX_NO_BANK exclude each other");
  if (pool && (qbar || wbar))
    return fail(DSAIDX_ERR_INVALID_ARG, "DSAIDX_POOL_MEAN takes NULL qbar and wbar");
  if (pool && Hs != H) return fail(DSAIDX_ERR_INVALID_ARG, "DSAIDX_POOL_MEAN needs Hs == H");
  if (Hs < 1) return fail(DSAIDX_ERR_INVALID_ARG, "Hs = %d must be positive", Hs);
  if (Hs > kMaxHeads) return fail(DSAIDX_ERR_UNSUPPORTED, "Hs = %d above %d", Hs, kMaxHeads);
  if (B > 0 && (!q || !k_cache || !k_scale || !w || !prefix_lens || !out_idx ||
                (!pool && !no_bank && (!qbar || !wbar))))
    return fail(DSAIDX_ERR_INVALID_ARG, "null q, k_cache, k_scale, w, qbar, wbar, prefix_lens or out_idx");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(w) || !aligned16(qbar) || !aligned16(wbar) ||
      !aligned16(out_idx) || !aligned16(out_score) || !aligned16(out_bank))
    return fail(DSAIDX_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (((uintptr_t)k_scale & 3u) || ((uintptr_t)prefix_lens & 3u))
    return fail(DSAIDX_ERR_INVALID_ARG, "k_scale and prefix_lens must be 4-byte aligned");
  const MtpWs lay = mtp_ws(B, Nmax, m, H, Hs, d, G, P, flags, out_bank == nullptr);
  rc = check_ws(ws, ws_bytes, lay.total);
  if (rc) return rc;
  if (B == 0) return ok();

  hipStream_t st = (hipStream_t)stream;
  uint8_t* base = (uint8_t*)ws;
  const int NGs = m / G;
  const int na = B * NGs, nr = B * m;
  MtpArgs t{};
  t.kc = k_cache;
  t.ks = k_scale;
  t.prefix = prefix_lens;
  t.B = B;
  t.m = m;
  t.G = G;
  t.P = P;
  t.d = d;
  t.Nmax = Nmax;
  t.a_kc = (const uint8_t**)(base + lay.a_kc);
  t.a_ks = (const float**)(base + lay.a_ks);
  t.a_len = (int32_t*)(base + lay.a_len);
  t.r_kc = (const uint8_t**)(base + lay.r_kc);
  t.r_ks = (const float**)(base + lay.r_ks);
  t.r_len_bank = (int32_t*)(base + lay.r_len);
  t.r_len_fb = (int32_t*)(base + lay.r_len2);
  int32_t* bank = out_bank ? out_bank : (int32_t*)(base + lay.bank);
  t.bank = bank;
  t.gk = base + lay.gk;
  t.gs = (float*)(base + lay.gs);
  t.out_idx = out_idx;
  t.topk = topk;
  t.no_bank = no_bank;
  hipError_t e = launch_mtp_plan(t, st);
  if (e != hipSuccess) return hip_fail(e, "indexer_mtp plan launch");

  // the group query of every group (windows that fall back never read it)
  const void* gq = qbar;
  const float* gw = wbar;
  if (pool) {
    PoolArgs pa{};
    pa.q = q;
    pa.w = w;
    pa.H = H;
    pa.d = d;
    pa.G = G;
    pa.g0 = 0;
    pa.ngroups = na;
    pa.qbar = base + lay.pq;
    pa.wbar = (float*)(base + lay.pw);
    gq = pa.qbar;
    gw = pa.wbar;
    e = launch_pool_mean(pa, st);
    if (e != hipSuccess) return hip_fail(e, "indexer_mtp pooling launch");
  }

  // 1. anchor scan: row (b, g) ranks its anchor's N + gG visible keys with
  //    the group indexer and keeps the best P, ascending (Eq. (8), (13));
  //    rows of windows that fall back have no keys and come out all -1
  DecodeArgs aa = decode_args(gq, gw, t.a_len, na, Nmax, Hs, d, P, base + lay.dec, bank, nullptr,
                              mtp_anchor_rows(B, m, Hs, G));
  aa.row_kc = t.a_kc;
  aa.row_ks = t.a_ks;
  e = launch_decode(aa, st);
  if (e != hipSuccess) return hip_fail(e, "indexer_mtp anchor scan launch");

  // 2. each bank group's candidates, bank then post-anchor keys, side by side
  e = launch_mtp_gather(t, st);
  if (e != hipSuccess) return hip_fail(e, "indexer_mtp gather launch");

  // 3. refinement of bank rows (Eq. (14)) over at most P + G - 1 candidates,
  //    and the original indexer for the rows of fallback windows; each launch
  //    leaves the other's rows (length -1) alone
  const int64_t cand = (int64_t)P + G - 1;
  DecodeArgs ar = decode_args(q, w, t.r_len_bank, nr, cand, H, d, topk, base + lay.dec, out_idx, out_score);
  ar.row_kc = t.r_kc;
  ar.row_ks = t.r_ks;
  ar.skip_negative = 1;
  e = launch_decode(ar, st);
  if (e != hipSuccess) return hip_fail(e, "indexer_mtp refine launch");
  DecodeArgs af = decode_args(q, w, t.r_len_fb, nr, Nmax, H, d, topk, base + lay.dec, out_idx, out_score);
  af.row_kc = t.r_kc;
  af.row_ks = t.r_ks;
  af.skip_negative = 1;
  e = launch_decode(af, st);
  if (e != hipSuccess) return hip_fail(e, "indexer_mtp fallback launch");

  // 4. bank rows: gathered positions -> token indices
  e = launch_mtp_map(t, st);
  if (e != hipSuccess) return hip_fail(e, "indexer_mtp map launch");
  return ok();
}

// ---------------------------------------------------- group query (Eq. 6-7)

struct GroupQueryWs {
  size_t pc, ph, cbar, qf, total;
};

static GroupQueryWs group_query_ws(int64_t Tq, int dc, int dh, int Hs, int d, int G) {
  const size_t n = (size_t)(Tq / G);
  GroupQueryWs w{};
  w.pc = 0;
  w.ph = w.pc + align_up(n * 3 * dc * 2u);
  w.cbar = w.ph + align_up(n * dh * 2u);
  w.qf = w.cbar + align_up(n * dc * 2u);
  w.total = w.qf + align_up(n * (size_t)Hs * d * 4u);
  return w;
}

size_t indexer_group_query_workspace_size(int64_t Tq, int dc, int dh, int Hs, int d, int G) {
  if (Tq <= 0 || dc <= 0 || dh <= 0 || Hs <= 0 || d <= 0 || G <= 0) return 0;
  return group_query_ws(Tq, dc, dh, Hs, d, G).total;
}

int indexer_group_query(const void* c, const void* h, const void* w_pool, const void* w_q,
                        const void* w_g, int64_t Tq, int dc, int dh, int Hs, int d, int G,
                        int64_t q_pos0, int rope_dim, float rope_base, void* qbar, float* wbar,
                        void* ws, size_t ws_bytes, void* stream) {
  if (Tq < 0 || q_pos0 < 0 || dc < 1 || dh < 1 || Hs < 1 || d < 1)
    return fail(DSAIDX_ERR_INVALID_ARG, "bad size (Tq=%lld dc=%d dh=%d Hs=%d d=%d)", (long long)Tq, dc,
                dh, Hs, d);
  if (G != 4 && G != 8 && G != 16)
    return fail(DSAIDX_ERR_UNSUPPORTED, "group size G = %d not in {4, 8, 16}", G);
  if (dc % 16 || dh % 16 || d % 16)
    return fail(DSAIDX_ERR_UNSUPPORTED, "dc, dh and d must be multiples of 16");
  if (Hs > kMaxHeads || (int64_t)Hs * d > 65536)
    return fail(DSAIDX_ERR_UNSUPPORTED, "Hs = %d, d = %d too large", Hs, d);
  if (dc > 65536 || dh > 65536) return fail(DSAIDX_ERR_UNSUPPORTED, "dc or dh above 65536");
  if (rope_dim < 0 || rope_dim > d || rope_dim % 2)
    return fail(DSAIDX_ERR_INVALID_ARG, "rope_dim = %d must be even and at most d", rope_dim);
  if (!(rope_base > 1.0f)) return fail(DSAIDX_ERR_INVALID_ARG, "rope_base must exceed 1");
  if (Tq / G > 65535) return fail(DSAIDX_ERR_UNSUPPORTED, "more than 65535 groups per call");
  if (Tq > 0 && (!c || !h || !w_pool || !w_q || !w_g || !qbar || !wbar))
    return fail(DSAIDX_ERR_INVALID_ARG, "null input or output");
  if (!aligned16(c) || !aligned16(h) || !aligned16(w_pool) || !aligned16(w_q) || !aligned16(w_g) ||
      ((uintptr_t)qbar & 1u) || ((uintptr_t)wbar & 3u))
    return fail(DSAIDX_ERR_INVALID_ARG, "inputs must be 16-byte aligned");
  const GroupQueryWs lay = group_query_ws(Tq, dc, dh, Hs, d, G);
  int rc = check_ws(ws, ws_bytes, lay.total);
  if (rc) return rc;
  if (Tq == 0) return ok();
  uint8_t* base = (uint8_t*)ws;
  GroupQueryArgs a{};
  a.c = c;
  a.h = h;
  a.w_pool = w_pool;
  a.w_q = w_q;
  a.w_g = w_g;
  a.dc = dc;
  a.dh = dh;
  a.Hs = Hs;
  a.d = d;
  a.G = G;
  a.rope_dim = rope_dim;
  a.rope_base = rope_base;
  a.q_pos0 = q_pos0;
  a.ngroups = Tq / G;
  a.tail = Tq % G != 0;
  a.pc = base + lay.pc;
  a.ph = base + lay.ph;
  a.cbar = base + lay.cbar;
  a.qf = (float*)(base + lay.qf);
  a.qbar = qbar;
  a.wbar = wbar;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (a.tail)  // the incomplete last group's gates are zero (its query row is zeroed by the kernel)
    e = launch_fill_i32((int32_t*)(wbar + a.ngroups * Hs), Hs, 0, st);
  if (e == hipSuccess) e = launch_group_query(a, st);
  if (e != hipSuccess) return hip_fail(e, "indexer_group_query launch");
  return ok();
}

// --------------------------------------------------------- calibration

int indexer_union_sizes(const int32_t* topk_idx, int64_t T, int K, int G, int32_t* out_union,
                        void* stream) {
  if (T < 0 || K < 1 || G < 1)
    return fail(DSAIDX_ERR_INVALID_ARG, "bad size (T=%lld K=%d G=%d)", (long long)T, K, G);
  if (G > 64) return fail(DSAIDX_ERR_UNSUPPORTED, "group size G = %d above 64", G);
  if (K > kMaxBank) return fail(DSAIDX_ERR_UNSUPPORTED, "K = %d above %d", K, kMaxBank);
  const int64_t groups = T / G;
  if (groups > INT32_MAX) return fail(DSAIDX_ERR_UNSUPPORTED, "too many groups");
  if (groups > 0 && (!topk_idx || !out_union))
    return fail(DSAIDX_ERR_INVALID_ARG, "null topk_idx or out_union");
  if (((uintptr_t)topk_idx & 15u) || ((uintptr_t)out_union & 3u))
    return fail(DSAIDX_ERR_INVALID_ARG, "topk_idx must be 16-byte aligned, out_union 4-byte");
  if (K % 4) return fail(DSAIDX_ERR_UNSUPPORTED, "K = %d is not a multiple of 4", K);
  const hipError_t e = launch_union_sizes(topk_idx, groups, K, G, out_union, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "indexer_union_sizes launch");
  return ok();
}

int indexer_topk_overlap(const int32_t* a, const int32_t* b, int64_t n, int K, int32_t* out_count,
                         void* stream) {
  if (n < 0 || K < 1) return fail(DSAIDX_ERR_INVALID_ARG, "bad size (n=%lld K=%d)", (long long)n, K);
  if (K > kMaxBank) return fail(DSAIDX_ERR_UNSUPPORTED, "K = %d above %d", K, kMaxBank);
  if (n > INT32_MAX) return fail(DSAIDX_ERR_UNSUPPORTED, "too many rows");
  if (n > 0 && (!a || !b || !out_count)) return fail(DSAIDX_ERR_INVALID_ARG, "null a, b or out_count");
  if (((uintptr_t)a & 15u) || ((uintptr_t)b & 3u) || ((uintptr_t)out_count & 3u))
    return fail(DSAIDX_ERR_INVALID_ARG, "a must be 16-byte aligned, b and out_count 4-byte");
  if (K % 4) return fail(DSAIDX_ERR_UNSUPPORTED, "K = %d is not a multiple of 4", K);
  const hipError_t e = launch_topk_overlap(a, b, n, K, out_count, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "indexer_topk_overlap launch");
  return ok();
}

int indexer_read_probe(const void* p, int64_t bytes, uint32_t* out, int nblocks, void* stream) {
  if (bytes < 0 || nblocks < 1 || nblocks > 65535)
    return fail(DSAIDX_ERR_INVALID_ARG, "bad size (bytes=%lld nblocks=%d)", (long long)bytes, nblocks);
  if (!out || (bytes > 0 && !p)) return fail(DSAIDX_ERR_INVALID_ARG, "null p or out");
  if (!aligned16(p) || ((uintptr_t)out & 3u))
    return fail(DSAIDX_ERR_INVALID_ARG, "p must be 16-byte aligned, out 4-byte");
  const hipError_t e = launch_read_probe(p, bytes, out, nblocks, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "indexer_read_probe launch");
  return ok();
}

int indexer_mfma_probe(int dtype, int iters, int waves_per_simd, int nblocks, uint32_t operand_mask, float* out,
                       uint64_t* clocks, void* stream) {
  if (dtype != DSAIDX_BF16 && dtype != DSAIDX_FP8_E4M3)
    return fail(DSAIDX_ERR_INVALID_ARG, "dtype %d is not DSAIDX_BF16 or DSAIDX_FP8_E4M3", dtype);
  if (iters < 1 || nblocks < 1 || nblocks > 65535)
    return fail(DSAIDX_ERR_INVALID_ARG, "bad size (iters=%d nblocks=%d)", iters, nblocks);
  if (waves_per_simd != 1 && waves_per_simd != 2 && waves_per_simd != 4)
    return fail(DSAIDX_ERR_INVALID_ARG, "waves_per_simd must be 1, 2 or 4 (got %d)", waves_per_simd);
  if (!out || !clocks) return fail(DSAIDX_ERR_INVALID_ARG, "null out or clocks");
  if (((uintptr_t)out & 3u) || ((uintptr_t)clocks & 7u))
    return fail(DSAIDX_ERR_INVALID_ARG, "out must be 4-byte aligned, clocks 8-byte");
  if (dtype == DSAIDX_FP8_E4M3) {
    // E4M3 NaN is S.1111.111: each mask byte must clear one of the low seven
    // bits, so that every operand is a number
    for (int k = 0; k < 4; ++k)
      if (((operand_mask >> (8 * k)) & 0x7Fu) == 0x7Fu)
        return fail(DSAIDX_ERR_INVALID_ARG, "operand_mask 0x%08x lets E4M3 NaN bytes through", operand_mask);
  } else {
    // bf16 infinities and NaNs have every exponent bit set: each mask half
    // must clear one of them
    for (int k = 0; k < 2; ++k)
      if (((operand_mask >> (16 * k)) & 0x7F80u) == 0x7F80u)
        return fail(DSAIDX_ERR_INVALID_ARG, "operand_mask 0x%08x lets bf16 infinities and NaNs through",
                    operand_mask);
  }
  // the kernels' dtype codes are the ABI's (bf16 1, E4M3 2)
  const hipError_t e =
      launch_mfma_probe(dtype, iters, waves_per_simd, nblocks, operand_mask, out, clocks, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "indexer_mfma_probe launch");
  return ok();
}

double indexer_union_stat(const int32_t* sizes, int64_t n, int stat) {
  if (n <= 0 || !sizes || stat < 0 || stat > 2) return -1.0;
  if (stat == 1) {
    double sum = 0.0;
    for (int64_t i = 0; i < n; ++i) sum += sizes[i];
    return sum / (double)n;
  }
  std::vector<int32_t> v(sizes, sizes + n);
  // max, or the nearest-rank 90th percentile: the ceil(0.9 n)-th smallest
  const int64_t k = stat == 0 ? n - 1 : (int64_t)std::ceil(0.9 * (double)n) - 1;
  std::nth_element(v.begin(), v.begin() + k, v.end());
  return (double)v[k];
}

// Scoring counts of Appendix A (one score = one unit, whatever the head count)
static double cost_pre_base(double L) { return 0.5 * L * L; }  // Eq. (15)
static double cost_pre_reuse(double L, int G, int P) {           // Eq. (19)
  if (L <= P) return cost_pre_base(L);
  return 0.5 * (double)P * P + (L * L - (double)P * P) / (2.0 * G) + (P + 0.5 * (G - 1)) * (L - P);
}
static double cost_mtp_base(double N, int m) { return m * N + 0.5 * m * (m - 1); }  // Eq. (16)
static double cost_mtp_reuse(double N, int G, int P, int m) {                       // Eq. (20)-(21)
  if (N <= P) return cost_mtp_base(N, m);
  double c = 0.0;
  for (int b = 0; b < m / G; ++b) c += N + (double)b * G + (double)G * P + 0.5 * G * (G - 1);
  return c;
}
// prefill of L tokens plus R verification rounds whose first query sees
// L + (j-1) a keys (Eq. (28)); G == 0 is the original indexer
static void cost_joint(double L, int G, int P, int R, int m, double a, double& base, double& reuse) {
  base = cost_pre_base(L);
  reuse = G ? cost_pre_reuse(L, G, P) : cost_pre_base(L);
  for (int j = 0; j < R; ++j) {
    const double N = L + j * a;
    base += cost_mtp_base(N, m);
    reuse += G ? cost_mtp_reuse(N, G, P, m) : cost_mtp_base(N, m);
  }
}

double indexer_speedup_joint(double L, int G, int P, int R, int m, double a) {
  if (L <= 0 || G < 1 || P < 1 || R < 0 || m < 1 || m % G || a < 0) return -1.0;
  double base, reuse;
  cost_joint(L, G, P, R, m, a, base, reuse);
  return base / reuse;
}

int indexer_select_setting(const double* stat_by_G, double L, int R, int m, double a, int* out_G,
                           int* out_P) {
  if (!stat_by_G || !out_G || !out_P) return fail(DSAIDX_ERR_INVALID_ARG, "null argument");
  if (L <= 0 || R < 0 || m < 16 || m % 16 || a < 0)
    return fail(DSAIDX_ERR_INVALID_ARG, "bad workload (L, R, m, a)");
  static const int kG[3] = {4, 8, 16}, kP[3] = {4096, 8192, 16384};
  double best = -1.0;
  *out_G = 0;
  *out_P = 0;
  for (int gi = 0; gi < 3; ++gi)
    for (int pi = 0; pi < 3; ++pi) {
      if (stat_by_G[gi] > kP[pi]) continue;  // Eq. (5): the bank must hold the statistic
      const double sp = indexer_speedup_joint(L, kG[gi], kP[pi], R, m, a);
      if (sp > best) {
        best = sp;
        *out_G = kG[gi];
        *out_P = kP[pi];
      }
    }
  return ok();
}

double indexer_layerwise_speedup(const int* G, const int* P, int nlayers, double L, int R, int m,
                                 double a) {
  if (nlayers <= 0 || !G || !P || L <= 0 || R < 0 || m < 1 || a < 0) return -1.0;
  double tb = 0.0, tr = 0.0;  // Eq. (27): counts summed over layers
  for (int i = 0; i < nlayers; ++i) {
    if (G[i] < 0 || (G[i] > 0 && (P[i] < 1 || m % G[i]))) return -1.0;
    double base, reuse;
    cost_joint(L, G[i], P[i], R, m, a, base, reuse);
    tb += base;
    tr += reuse;
  }
  return tb / tr;
}

}  // extern "C"
