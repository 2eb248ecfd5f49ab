// mtp.hip -- the glue kernels of MTP target verification (ADIndex (Qi et
// al.), Section 4.3 "Application to Prefill and MTP", Appendix A.2).
//
// Each of B sequences verifies a window of m queries; query r sits at
// position N - 1 + r of its sequence (it sees N + r keys), N = prefix[b].  A
// window reuses banks only when N > P (one decision per window): group g's
// anchor (query gG) ranks its N + gG visible keys with the group indexer and
// keeps the best P (the bank); member i of the group then ranks the bank plus
// the i keys after the anchor with its own query.  Windows with N <= P use
// the original indexer for all m queries.
//
// Both scans are the decode pipeline (one query per row against a key
// sequence, decode.hip) run over "rows": the anchor scan has one row per
// (sequence, group) over the sequence's cache; the refinement has one row per
// query, over the gathered candidates of its group (bank rows) or over its
// sequence's cache (fallback rows).  Bank rows and fallback rows are refined
// by two launches, each sized for its own row length (about P, or up to
// Nmax); a row owned by the other launch has length -1 and is left alone.  These kernels set those rows up, gather
// each bank group's candidate keys -- the bank, then the G-1 keys after the
// anchor, already ascending -- into one contiguous run, and map refinement
// output positions back to token indices (monotone, so the tie order of equal
// scores, lower index first, carries over).
#include "device.h"
#include "launch.h"

namespace dsaidx {

namespace {

constexpr int kMtpThreads = 256;

__device__ __forceinline__ int64_t window_start(const MtpArgs& a, int b) {
  int64_t n = a.prefix[b];
  const int64_t hi = a.Nmax - a.m + 1;
  return n < 1 ? 1 : (n > hi ? hi : n);
}

// the window reuses banks: its first query sees more than P keys (and the
// caller did not ask for the original indexer throughout)
__device__ __forceinline__ bool uses_bank(const MtpArgs& a, int64_t N) { return !a.no_bank && N > a.P; }

__global__ void __launch_bounds__(kMtpThreads) mtp_plan_kernel(const MtpArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * kMtpThreads + threadIdx.x;
  const int NGs = a.m / a.G;
  const int64_t cand = (int64_t)a.P + a.G - 1;  // gathered keys per bank group
  if (idx < (int64_t)a.B * NGs) {
    const int b = (int)(idx / NGs), g = (int)(idx % NGs);
    const int64_t N = window_start(a, b);
    a.a_kc[idx] = a.kc + (int64_t)b * a.Nmax * a.d;
    a.a_ks[idx] = a.ks + (int64_t)b * a.Nmax;
    a.a_len[idx] = uses_bank(a, N) ? (int32_t)(N + (int64_t)g * a.G) : 0;
  }
  if (idx < (int64_t)a.B * a.m) {
    const int b = (int)(idx / a.m), r = (int)(idx % a.m);
    const int g = r / a.G, i = r % a.G;
    const int64_t N = window_start(a, b);
    if (uses_bank(a, N)) {
      const int64_t grp = (int64_t)b * NGs + g;
      a.r_kc[idx] = a.gk + grp * cand * a.d;
      a.r_ks[idx] = a.gs + grp * cand;
      a.r_len_bank[idx] = a.P + i;
      a.r_len_fb[idx] = -1;
    } else {
      a.r_kc[idx] = a.kc + (int64_t)b * a.Nmax * a.d;
      a.r_ks[idx] = a.ks + (int64_t)b * a.Nmax;
      a.r_len_bank[idx] = -1;
      a.r_len_fb[idx] = (int32_t)(N + r);
    }
  }
}

// token index of gathered position p of bank group (b, g)
__device__ __forceinline__ int32_t gathered_token(const MtpArgs& a, int64_t grp, int64_t anchor, int64_t p) {
  return p < a.P ? a.bank[grp * a.P + p] : (int32_t)(anchor + 1 + (p - a.P));
}

// blockIdx.y = bank group; each thread copies one 16-byte chunk of a key row
// (and the row's scale); 256 threads cover 256*16/d rows.
__global__ void __launch_bounds__(kMtpThreads) mtp_gather_kernel(const MtpArgs a) {
  const int NGs = a.m / a.G;
  const int64_t grp = blockIdx.y;
  const int b = (int)(grp / NGs), g = (int)(grp % NGs);
  const int64_t N = window_start(a, b);
  if (!uses_bank(a, N)) return;  // this window falls back: nothing to gather
  const int64_t anchor = N - 1 + (int64_t)g * a.G;
  const int cpr = a.d / 16;  // chunks per key row
  const int rows_per_block = kMtpThreads / cpr;
  const int64_t cand = (int64_t)a.P + a.G - 1;
  const int64_t p = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / cpr;
  const int c = threadIdx.x % cpr;
  if (p >= cand) return;
  const int32_t tok = gathered_token(a, grp, anchor, p);
  const uint8_t* src_row = a.kc + ((int64_t)b * a.Nmax + (tok < 0 ? 0 : tok)) * a.d;
  uint4 v = tok < 0 ? make_uint4(0, 0, 0, 0) : reinterpret_cast<const uint4*>(src_row)[c];
  reinterpret_cast<uint4*>(a.gk + (grp * cand + p) * a.d)[c] = v;
  if (c == 0) a.gs[grp * cand + p] = tok < 0 ? 0.0f : a.ks[(int64_t)b * a.Nmax + tok];
}

// blockIdx.y = refinement row; positions of bank rows become token indices
__global__ void __launch_bounds__(kMtpThreads) mtp_map_kernel(const MtpArgs a) {
  const int64_t row = blockIdx.y;
  const int b = (int)(row / a.m), r = (int)(row % a.m);
  const int64_t N = window_start(a, b);
  if (!uses_bank(a, N)) return;  // fallback rows already hold token indices
  const int j = blockIdx.x * kMtpThreads + threadIdx.x;
  if (j >= a.topk) return;
  const int g = r / a.G;
  const int64_t grp = (int64_t)b * (a.m / a.G) + g;
  const int64_t anchor = N - 1 + (int64_t)g * a.G;
  int32_t* o = a.out_idx + row * a.topk + j;
  const int32_t p = *o;
  if (p >= 0) *o = gathered_token(a, grp, anchor, p);
}

}  // namespace

hipError_t launch_mtp_plan(const MtpArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.B * a.m;  // >= B * m/G
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(mtp_plan_kernel, dim3((unsigned)((n + kMtpThreads - 1) / kMtpThreads)),
                     dim3(kMtpThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mtp_gather(const MtpArgs& a, hipStream_t stream) {
  const int64_t groups = (int64_t)a.B * (a.m / a.G);
  if (groups <= 0) return hipSuccess;
  const int rows_per_block = kMtpThreads / (a.d / 16);
  const int64_t cand = (int64_t)a.P + a.G - 1;
  hipLaunchKernelGGL(mtp_gather_kernel,
                     dim3((unsigned)((cand + rows_per_block - 1) / rows_per_block), (unsigned)groups),
                     dim3(kMtpThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mtp_map(const MtpArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.m;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(mtp_map_kernel, dim3((unsigned)((a.topk + kMtpThreads - 1) / kMtpThreads), (unsigned)rows),
                     dim3(kMtpThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsaidx
