// noalloc.hip -- the decode indexer for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc): indexer_decode with its workspace in a file-scope device array
// of fixed size instead of a caller buffer.
//
// The array is a device symbol: each GPU the library runs on holds its own
// copy at its own address from the library's load until the process ends.
// Host code never uses the array's name as an address (on the host it is a
// stand-in, and passing it to a kernel faults); it asks the runtime for the
// current device's address once per device and passes that pointer as the
// decode pipeline's workspace.  Calls that overlap on one GPU share the array
// and race; the pipeline clears every part of it that must start at zero, on
// the stream, at the start of each call.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "dsa_indexer.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = size_t(96) << 20;  // 96 MiB: 32 sequences x 256K keys need 68.6 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // the device address of `scratch` on each device, once looked up

// The scratch array's address on `dev` (the current device), looked up on the
// first call for that device.  Returns nullptr and sets the error on failure.
void* scratch_on(int dev, int* rc) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *rc = dsaidx::report_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                     "indexer_decode_noalloc: scratch address");
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t indexer_decode_noalloc_max_bytes(void) { return kScratchBytes; }

int indexer_decode_noalloc(const void* q, const uint8_t* k_cache, const float* k_scale, const float* w,
                           const int32_t* seq_lens, int B, int64_t Nmax, int H, int d, int topk,
                           int32_t* out_idx, float* out_score, void* stream) {
  const size_t need = indexer_decode_workspace_size(B, Nmax, H, d, topk);
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "indexer_decode_noalloc: B=%d x Nmax=%lld needs %zu bytes of scratch, above its fixed %zu "
             "(use indexer_decode with a workspace)",
             B, (long long)Nmax, need, kScratchBytes);
    return dsaidx::report_error(DSAIDX_ERR_UNSUPPORTED, msg);
  }
  void* ws = nullptr;
  if (need > 0) {
    // the stream's device (the current device for the null stream)
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return dsaidx::report_hip_error(e, "indexer_decode_noalloc: device of the stream");
    if (dev < 0 || dev >= kMaxDevices)
      return dsaidx::report_error(DSAIDX_ERR_UNSUPPORTED, "indexer_decode_noalloc: device index above 63");
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return dsaidx::report_hip_error(e, "indexer_decode_noalloc: current device");
    if (cur != dev)
      return dsaidx::report_error(DSAIDX_ERR_INVALID_ARG,
                                  "indexer_decode_noalloc: the stream's device is not the current device");
    int rc = DSAIDX_OK;
    ws = scratch_on(dev, &rc);
    if (!ws) return rc;
  }
  // argument checks, then the same kernels as indexer_decode, on the scratch
  return indexer_decode(q, k_cache, k_scale, w, seq_lens, B, Nmax, H, d, topk, out_idx, out_score, ws,
                        need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"
