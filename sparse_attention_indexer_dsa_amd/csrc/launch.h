// launch.h -- host-side launchers of the indexer kernels (internal to libdsaidx).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsaidx {

// One launch of the streaming score + top-K kernel over `nq` query rows.
// Row j sits at position pos0 + j * pos_stride.  With bank == nullptr the
// candidates of row j are keys 0 .. its position; otherwise the launch's rows
// form consecutive groups of `group` (nq a multiple of 4 and of group) and the
// candidates of row j are its group's bank (bank + g * bank_stride, the first
// min(bank_stride, anchor+1) entries, ascending) followed by anchor+1 .. its
// position, where anchor = pos0 + g * group.
struct ScanArgs {
  const void* q;         // [nq, H, d] bf16 or E4M3
  const float* q_scale;  // [nq] (E4M3) or nullptr
  const float* w;        // [nq, H]
  const void* k;         // [Tk, d]
  const float* k_scale;  // [Tk] (E4M3) or nullptr
  int H, d;
  int64_t nq, pos0;
  int pos_stride;
  const int32_t* bank;
  int bank_stride, group;
  int K, cap;              // top-K; candidate-buffer entries per row (>= 2K + 2048, < 65536)
  uint32_t* cand_key;      // [nq, cap] workspace
  int32_t* cand_idx;       // [nq, cap] workspace
  int32_t* out_idx;        // [nq, out_stride]
  float* out_score;        // [nq, out_stride] or nullptr
  int out_stride;
  // Sampled start of the dense E4M3 kernel over contiguous keys (nullptr:
  // none): start [nq] floats, rerun [ceil(nq / 8)] flags, both workspace.
  // rerun_pass is set inside the launch; sample_test != 0 puts every start
  // above all scores, so that each sampled workgroup is streamed a second
  // time (a test of that path; the results are the same).
  float* start;
  int32_t* rerun;
  int rerun_pass;
  int sample_test;
};

hipError_t launch_scan_topk(const ScanArgs& a, int dtype, hipStream_t stream);

// The dense kernel for 33..64 heads at d = 128 (bank groups: a multiple of 8
// queries, pos_stride 1); launch_scan_topk routes there when
// dense_topk_supported().
bool dense_topk_supported(const ScanArgs& a);
hipError_t launch_dense_topk(const ScanArgs& a, int dtype, hipStream_t stream);

// Row histogram of the decode scores: bins of the top kDecHistBits bits of the
// order-preserving key.
constexpr int kDecHistBits = 12;
constexpr int kDecHistBins = 1 << kDecHistBits;

// Decode: scores of one bf16 query per sequence against its E4M3 cache, then
// a per-row top-K.  Scan workgroups cover kpb keys of a row each and keep, in
// a compact list, only the scores that can still reach the row's top K.  The
// list is stored as kDecListSegs segments, one per wave of the workgroup: the
// kpb slots of span j hold segment w (the kept keys of the span's w-th
// quarter, ascending) at slots w*kpb/kDecListSegs onwards, and cl_cnt holds
// each segment's count; read in segment order the list is ascending.
constexpr int kDecListSegs = 4;
struct DecodeArgs {
  const void* q;          // [B, H, d] bf16
  const uint8_t* kc;      // [B, Nmax, d] E4M3
  const float* k_scale;   // [B, Nmax]
  const float* w;         // [B, H]
  const int32_t* seq_lens;  // [B]
  // optional per-row key sources (row b reads row_kc[b] [.., d] and
  // row_ks[b]); when null, row b reads kc + b*Nmax*d and k_scale + b*Nmax
  const uint8_t* const* row_kc;
  const float* const* row_ks;
  int skip_negative;  // rows with seq_lens < 0 write nothing (else: clamped to 0)
  // rows per scan workgroup (1, 2 or 4; see dec_scan_rows_ok): rows rR .. rR+R-1
  // share row r*R's key source and are scored in one pass over it
  int scan_rows;
  int B, H, d;
  int64_t Nmax;
  int K;
  int64_t kpb;            // keys per scan workgroup: a multiple of 256, <= dec_max_kpb(scan_rows)
  int nblk;               // scan workgroups per row: ceil(Nmax / kpb)
  uint32_t* hist;         // [B, kDecHistBins] workspace, zeroed per call
  int32_t* cl_cnt;        // [B, nblk, kDecListSegs] entries of each list segment
  int32_t* cl_idx;        // [B, nblk, kpb] key indices of the compact lists (segments)
  float* cl_sc;           // [B, nblk, kpb] their scores
  int32_t* cand_cnt;      // [B] threshold-bin candidates gathered, zeroed per call
  uint32_t* cand_key;     // [B, kDecCandCap] their order keys
  int32_t* cand_idx;      // [B, kDecCandCap] their key indices
  int32_t* span_above;    // [B, nblk] list entries above the threshold bin
  int32_t* span_off;      // [B, nblk] output offset of each span's selected keys
  uint32_t* rowsel;       // [B, 4] emission: mode (1 = by span), K-th key, tie cut
  int32_t* out_idx;       // [B, K]
  float* out_score;       // [B, K] or nullptr
};
constexpr int kDecKeysPerPass = 768;  // keys one scan workgroup scores per loop trip
constexpr int kDecMaxKpb = 16384;     // keys per scan workgroup at most (its LDS score stage)
// keys per scan workgroup at most when it scores R rows (R LDS score stages)
constexpr int dec_max_kpb(int R) { return R == 1 ? kDecMaxKpb : kDecMaxKpb / 2 / R; }
// Several rows per scan workgroup: 8 heads per row (R rows fill 8R MFMA rows),
// R in {2, 4}, and the rows of a workgroup must share one key source.
constexpr bool dec_scan_rows_ok(int R, int H, int B) { return (R == 2 || R == 4) && H == 8 && B % R == 0; }
constexpr int kDecCandCap = 16384;    // threshold-bin candidates a row keeps in LDS

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);


// Mean-pooled group query: for groups g0 .. g0+ngroups-1 of G consecutive
// queries of q [*, H, d] bf16 and w [*, H], writes qbar [ngroups, H, d] bf16
// and wbar [ngroups, H] fp32 (fp32 sums in query order, times 1/G, q rounded
// to the nearest bf16).  H*d a multiple of 8, q 16-byte aligned; H <= 256.
struct PoolArgs {
  const void* q;
  const float* w;
  int H, d, G;
  int64_t g0, ngroups;
  void* qbar;
  float* wbar;
};
hipError_t launch_pool_mean(const PoolArgs& a, hipStream_t stream);

// MTP verification windows (B sequences, m queries each, groups of G, bank P):
// per-row key sources and lengths for the anchor scan (rows b*NGs + g) and the
// refinement (rows b*m + r), the gathered candidate keys of every bank group,
// and the map from refinement positions back to token indices.
struct MtpArgs {
  const uint8_t* kc;       // [B, Nmax, d] E4M3
  const float* ks;         // [B, Nmax]
  const int32_t* prefix;   // [B] keys the window's first query sees (clamped to [1, Nmax-m+1])
  int B, m, G, P, d;
  int64_t Nmax;
  const uint8_t** a_kc;  const float** a_ks;  int32_t* a_len;   // [B*m/G]
  const uint8_t** r_kc;  const float** r_ks;  // [B*m]
  int32_t* r_len_bank;     // [B*m] refinement lengths of bank rows, -1 elsewhere
  int32_t* r_len_fb;       // [B*m] lengths of fallback rows, -1 elsewhere
  const int32_t* bank;     // [B*m/G, P] ascending (anchor scan output)
  uint8_t* gk;             // [B*m/G, P+G-1, d] gathered keys
  float* gs;               // [B*m/G, P+G-1] their scales
  int32_t* out_idx;        // [B*m, topk] refinement output, mapped in place
  int topk;
  int no_bank;             // every window uses the original indexer
};
hipError_t launch_mtp_plan(const MtpArgs& a, hipStream_t stream);
hipError_t launch_mtp_gather(const MtpArgs& a, hipStream_t stream);
hipError_t launch_mtp_map(const MtpArgs& a, hipStream_t stream);

// The group indexer's query and gates (Eq. (6)-(7)) for `ngroups` complete
// groups of G rows of c [*, dc] and h [*, dh] (bf16), plus one zero row of
// qbar when `tail` (an incomplete last group).  Workspace: pc [ngroups, 3dc],
// ph [ngroups, dh], cbar [ngroups, dc] bf16; qf [ngroups, Hs*d] fp32.
struct GroupQueryArgs {
  const void* c;
  const void* h;
  const void* w_pool;  // [dc, 3dc]
  const void* w_q;     // [Hs*d, dc]
  const void* w_g;     // [Hs, dh]
  int dc, dh, Hs, d, G, rope_dim;
  float rope_base;
  int64_t q_pos0, ngroups;
  int tail;
  void* pc;
  void* ph;
  void* cbar;
  float* qf;
  void* qbar;   // [ngroups + tail, Hs, d] bf16
  float* wbar;  // [ngroups + tail, Hs]; the tail row is written by the caller
};
hipError_t launch_group_query(const GroupQueryArgs& a, hipStream_t stream);

// Calibration statistics over top-K index sets [rows, K] (ascending, -1 padded):
// the union size of each complete group of G rows, and per-row overlaps.
hipError_t launch_union_sizes(const int32_t* idx, int64_t groups, int K, int G, int32_t* out,
                              hipStream_t stream);
hipError_t launch_topk_overlap(const int32_t* a, const int32_t* b, int64_t n, int K, int32_t* out,
                               hipStream_t stream);

// Read `bytes` bytes at p once (coalesced 16-byte loads); out [nblocks] gets
// one XOR word per workgroup.
hipError_t launch_read_probe(const void* p, int64_t bytes, uint32_t* out, int nblocks, hipStream_t stream);
hipError_t launch_mfma_probe(int dtype, int iters, int waves_per_simd, int nblocks, uint32_t mask, float* out,
                             uint64_t* clocks, hipStream_t stream);

// Set the calling thread's last-error message (indexer_last_error) and return
// `code`; for entry points outside api.cpp.
int report_error(int code, const char* msg);
int report_hip_error(hipError_t e, const char* what);

// Fill n int32 values with v (a kernel, not a memset node).
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream);

}  // namespace dsaidx
