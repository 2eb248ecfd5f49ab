// group_query.hip -- the group indexer's query and gates of ADIndex (Qi et
// al.), Section 4.2 Eq. (6)-(7) and Appendix C.3:
//
//   cbar = W_pool [max_i c_i ; min_i c_i ; mean_i c_i],  hbar = mean_i h_i
//   qbar_j = RoPE_anchor([W_Q cbar]_j),  wbar_j = sigmoid([W_G hbar]_j)
//
// over each complete group of G consecutive query rows.  Pooling reads the
// latents and hidden states once (HBM-bound: the hidden states dominate); the
// two query products are plain bf16 matrix products with fp32 accumulation on
// the 32x32x16 bf16 MFMA, K contiguous in both operands, staged through LDS
// in chunks of 64 k; the gate's few heads are dot products;
// the rotary embedding (fp64 angles, the
// positions reach 10^5 radians) and the bf16 rounding of the query follow in
// their own small kernel.
#include "device.h"
#include "launch.h"

namespace dsaidx {

namespace {

constexpr int kGqThreads = 256;

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)bf16_rne(lo) | ((uint32_t)bf16_rne(hi) << 16);
}

// One thread per 8 columns of a group, of c (the first dc/8 threads) or of h
// (the next dh/8): max, min and mean of c's rows (into pc [n, 3dc]) or the
// mean of h's rows (into ph [n, dh]), fp32 sums in row order times 1/G,
// rounded to bf16.  Every thread has its G loads in flight together.
template <int G>
__global__ void __launch_bounds__(kGqThreads) gq_pool_kernel(const GroupQueryArgs a) {
  const int64_t g = blockIdx.y;
  const int cc = a.dc / 8, hc = a.dh / 8;  // 16-byte chunks per row
  const int xt = blockIdx.x * kGqThreads + threadIdx.x;
  const float inv = 1.0f / (float)G;
  if (xt < cc) {
    const int x = xt;
    const uint4* src = reinterpret_cast<const uint4*>(a.c) + g * G * cc + x;
    uint4 v[G];
#pragma unroll
    for (int i = 0; i < G; ++i) v[i] = src[(int64_t)i * cc];
    float mx[8], mn[8], s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) { mx[j] = -__builtin_inff(); mn[j] = __builtin_inff(); s[j] = 0.0f; }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float e0 = bf_lo(w[q]), e1 = bf_hi(w[q]);
        mx[2 * q] = fmaxf(mx[2 * q], e0); mx[2 * q + 1] = fmaxf(mx[2 * q + 1], e1);
        mn[2 * q] = fminf(mn[2 * q], e0); mn[2 * q + 1] = fminf(mn[2 * q + 1], e1);
        s[2 * q] += e0; s[2 * q + 1] += e1;
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(a.pc) + g * 3 * cc + x;
    dst[0] = make_uint4(pack_bf16(mx[0], mx[1]), pack_bf16(mx[2], mx[3]), pack_bf16(mx[4], mx[5]),
                        pack_bf16(mx[6], mx[7]));
    dst[cc] = make_uint4(pack_bf16(mn[0], mn[1]), pack_bf16(mn[2], mn[3]), pack_bf16(mn[4], mn[5]),
                         pack_bf16(mn[6], mn[7]));
    dst[2 * cc] = make_uint4(pack_bf16(s[0] * inv, s[1] * inv), pack_bf16(s[2] * inv, s[3] * inv),
                             pack_bf16(s[4] * inv, s[5] * inv), pack_bf16(s[6] * inv, s[7] * inv));
  } else if (xt < cc + hc) {
    const int x = xt - cc;
    const uint4* src = reinterpret_cast<const uint4*>(a.h) + g * G * hc + x;
    uint4 v[G];
#pragma unroll
    for (int i = 0; i < G; ++i) v[i] = src[(int64_t)i * hc];
    float s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) { s[2 * q] += bf_lo(w[q]); s[2 * q + 1] += bf_hi(w[q]); }
    }
    reinterpret_cast<uint4*>(a.ph)[g * hc + x] =
        make_uint4(pack_bf16(s[0] * inv, s[1] * inv), pack_bf16(s[2] * inv, s[3] * inv),
                   pack_bf16(s[4] * inv, s[5] * inv), pack_bf16(s[6] * inv, s[7] * inv));
  }
}

// C = A B^T for A [M, K], B [N, K] bf16 (K contiguous, K % 16 == 0), fp32
// accumulation.  A workgroup covers 128 x 128 of C and walks K in chunks of
// 64: each chunk of both operands (2 x 16 KB) is staged in LDS, double
// buffered, and the next chunk's global loads (eight 16-byte loads per
// thread, coalesced along K) are in flight while the current one is
// multiplied.  Each wave computes 64 x 64 as 2 x 2 tiles of the 32x32x16 bf16
// MFMA; lane l's A fragment of a tile and k-step is row l%32, k 8(l/32)..+7
// (one 16-byte LDS read), likewise for B; lane l then holds
// C[8(r/4) + 4(l/32) + r%4][l%32].  The MFMAs of every output tile run in
// ascending k.  Rows past M or N are clamped on load and skipped on store; k
// past K loads zeros.
// MODE 0: C bf16 [M, N]; 1: C fp32 [M, N].
constexpr int kGmTile = 128;                        // rows of C per workgroup (and columns)
constexpr int kGmKc = 64;                           // k per LDS chunk
constexpr int kGmRowBytes = kGmKc * 2;              // one operand row of a chunk: 8 x 16 B
constexpr int kGmMatBytes = kGmTile * kGmRowBytes;  // 16 KB per operand and chunk
// 16-byte chunk c of row r sits at slot c ^ ((r >> 1) & 7): any 16
// consecutive rows put one chunk in 16 distinct 16-byte bank groups
__device__ __forceinline__ int gm_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int MODE>
__global__ void __launch_bounds__(kGqThreads) gemm_nt_kernel(const uint16_t* A, const uint16_t* B, int M,
                                                             int N, int K, void* C) {
  __shared__ __attribute__((aligned(16))) uint8_t s_op[2][2 * kGmMatBytes];  // [buffer][A rows | B rows]
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int mb = blockIdx.y * kGmTile, nb = blockIdx.x * kGmTile;
  // this thread's eight chunks of a k-chunk: q = tid + 256i, A for q < 1024
  // (row q/8, chunk q%8), B after
  constexpr int kLoads = 2 * kGmMatBytes / 16 / kGqThreads;
  const uint16_t* src[kLoads];
  int soff[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int q = tid + kGqThreads * i;
    const int mat = q / (kGmTile * 8), row = (q / 8) % kGmTile, c = q % 8;
    const int lim = mat ? N : M;
    const int grow = min((mat ? nb : mb) + row, lim - 1);
    src[i] = (mat ? B : A) + (int64_t)grow * K + 8 * c;
    soff[i] = mat * kGmMatBytes + row * kGmRowBytes + 16 * gm_slot(row, c);
  }
  u32x4 st[kLoads];
  auto gload = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = (tid + kGqThreads * i) % 8;
      st[i] = k0 + 8 * c < K ? *reinterpret_cast<const u32x4*>(src[i] + k0) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) *reinterpret_cast<u32x4*>(&s_op[buf][soff[i]]) = st[i];
  };
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  v16f acc[2][2] = {};
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const uint8_t* sa = &s_op[buf][0];
    const uint8_t* sb = &s_op[buf][kGmMatBytes];
#pragma unroll
    for (int s = 0; s < kGmKc / 16; ++s) {
      const int c = 2 * s + (l >> 5);
      v8bf af[2], bf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ra = wm + 32 * t + (l & 31), rb = wn + 32 * t + (l & 31);
        af[t] = *reinterpret_cast<const v8bf*>(sa + ra * kGmRowBytes + 16 * gm_slot(ra, c));
        bf[t] = *reinterpret_cast<const v8bf*>(sb + rb * kGmRowBytes + 16 * gm_slot(rb, c));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };
  const int nk = (K + kGmKc - 1) / kGmKc;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const bool more = kc + 1 < nk;
    if (more) gload((kc + 1) * kGmKc);
    compute(kc & 1);
    if (more) lstore((kc + 1) & 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = nb + wn + 32 * j + (l & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mb + wm + 32 * i + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        if (row >= M) continue;
        const int64_t o = (int64_t)row * N + col;
        const float v = acc[i][j][r];
        if constexpr (MODE == 0) reinterpret_cast<uint16_t*>(C)[o] = bf16_rne(v);
        else reinterpret_cast<float*>(C)[o] = v;
      }
    }
}

// wbar = sigmoid(W_G hbar): one workgroup per 8 groups, 8 heads per pass.
// Thread t takes 8-column chunks t, t+256, ... of the groups' hbar rows and
// of the heads' W_G rows, each loaded once per pass (fp32 FMA, in chunk
// order), then a butterfly sum over the wave and a sum over the waves in
// order per (group, head): every wbar is summed as with one workgroup per
// group.
constexpr int kGateGroups = 8;
constexpr int kGateHeads = 8;
__global__ void __launch_bounds__(kGqThreads) gq_gate_kernel(const GroupQueryArgs a) {
  __shared__ float s_part[kGateHeads * kGateGroups][kGqThreads / 64];
  const int64_t g0 = (int64_t)blockIdx.x * kGateGroups;
  const int ng = a.ngroups - g0 < kGateGroups ? (int)(a.ngroups - g0) : kGateGroups;
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int hc = a.dh / 8;
  const uint4* hrows = reinterpret_cast<const uint4*>(a.ph) + g0 * hc;
  for (int j0 = 0; j0 < a.Hs; j0 += kGateHeads) {
    const int nh = a.Hs - j0 < kGateHeads ? a.Hs - j0 : kGateHeads;
    float acc[kGateHeads][kGateGroups];
#pragma unroll
    for (int jj = 0; jj < kGateHeads; ++jj)
#pragma unroll
      for (int gi = 0; gi < kGateGroups; ++gi) acc[jj][gi] = 0.0f;
    for (int x = tid; x < hc; x += kGqThreads) {
      uint4 hv[kGateGroups];
#pragma unroll
      for (int gi = 0; gi < kGateGroups; ++gi) hv[gi] = gi < ng ? hrows[gi * hc + x] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int jj = 0; jj < kGateHeads; ++jj) {
        if (jj >= nh) break;
        const uint4 wv = reinterpret_cast<const uint4*>(a.w_g)[(int64_t)(j0 + jj) * hc + x];
        const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int gi = 0; gi < kGateGroups; ++gi) {
          const uint32_t hw[4] = {hv[gi].x, hv[gi].y, hv[gi].z, hv[gi].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[jj][gi] = fmaf(bf_lo(hw[q]), bf_lo(ww[q]), acc[jj][gi]);
            acc[jj][gi] = fmaf(bf_hi(hw[q]), bf_hi(ww[q]), acc[jj][gi]);
          }
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < kGateHeads; ++jj)
#pragma unroll
      for (int gi = 0; gi < kGateGroups; ++gi) {
        float v = acc[jj][gi];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        if (l == 0) s_part[jj * kGateGroups + gi][wave] = v;
      }
    __syncthreads();
    if (tid < kGateHeads * kGateGroups) {
      const int jj = tid / kGateGroups, gi = tid % kGateGroups;
      if (jj < nh && gi < ng) {
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < kGqThreads / 64; ++w) t += s_part[tid][w];
        a.wbar[(g0 + gi) * a.Hs + j0 + jj] = 1.0f / (1.0f + __expf(-t));
      }
    }
    __syncthreads();
  }
}

// qbar rows: rotate the pairs (i, i + rope_dim/2) of every head at the
// group's anchor position, round to bf16; the incomplete last group's row
// is zero.  One thread per (group, head, pair-or-entry).
__global__ void __launch_bounds__(kGqThreads) gq_rope_kernel(const GroupQueryArgs a) {
  const int64_t g = blockIdx.y;
  const int HD = a.Hs * a.d;
  const int e = blockIdx.x * kGqThreads + threadIdx.x;  // entry of the row
  if (e >= HD) return;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.qbar) + g * HD;
  if (g >= a.ngroups) {  // the incomplete last group
    out[e] = 0;
    return;
  }
  const float* q = a.qf + g * HD;
  const int j = e / a.d, i = e % a.d, half = a.rope_dim / 2;
  float v = q[e];
  if (i < a.rope_dim) {
    const int p = i < half ? i : i - half;  // pair index
    const double pos = (double)(a.q_pos0 + g * a.G);
    const double ang = pos * pow((double)a.rope_base, -2.0 * p / a.rope_dim);
    const double cs = cos(ang), sn = sin(ang);
    const double x0 = q[j * a.d + p], x1 = q[j * a.d + p + half];
    v = (float)(i < half ? x0 * cs - x1 * sn : x1 * cs + x0 * sn);
  }
  out[e] = bf16_rne(v);
}

}  // namespace

hipError_t launch_group_query(const GroupQueryArgs& a, hipStream_t stream) {
  const int64_t n = a.ngroups;
  if (n > 0) {
    const int chunks = (a.dc + a.dh) / 8;
    const dim3 pg((unsigned)((chunks + kGqThreads - 1) / kGqThreads), (unsigned)n);
    switch (a.G) {
      case 4: hipLaunchKernelGGL(gq_pool_kernel<4>, pg, dim3(kGqThreads), 0, stream, a); break;
      case 8: hipLaunchKernelGGL(gq_pool_kernel<8>, pg, dim3(kGqThreads), 0, stream, a); break;
      case 16: hipLaunchKernelGGL(gq_pool_kernel<16>, pg, dim3(kGqThreads), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    auto grid = [&](int N) {
      return dim3((unsigned)((N + kGmTile - 1) / kGmTile), (unsigned)((n + kGmTile - 1) / kGmTile));
    };
    // cbar = W_pool [max; min; mean]        [n, dc]  (bf16: the next product's operand)
    hipLaunchKernelGGL(gemm_nt_kernel<0>, grid(a.dc), dim3(kGqThreads), 0, stream, (const uint16_t*)a.pc,
                       (const uint16_t*)a.w_pool, (int)n, a.dc, 3 * a.dc, (void*)a.cbar);
    // q = W_Q cbar                           [n, Hs*d] fp32
    hipLaunchKernelGGL(gemm_nt_kernel<1>, grid(a.Hs * a.d), dim3(kGqThreads), 0, stream,
                       (const uint16_t*)a.cbar, (const uint16_t*)a.w_q, (int)n, a.Hs * a.d, a.dc, (void*)a.qf);
    // wbar = sigmoid(W_G hbar)              [n, Hs] fp32 (Hs is small: dot products)
    hipLaunchKernelGGL(gq_gate_kernel, dim3((unsigned)((n + kGateGroups - 1) / kGateGroups)), dim3(kGqThreads), 0,
                       stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t rows = a.ngroups + (a.tail ? 1 : 0);
  if (rows > 0) {
    const int HD = a.Hs * a.d;
    hipLaunchKernelGGL(gq_rope_kernel, dim3((unsigned)((HD + kGqThreads - 1) / kGqThreads), (unsigned)rows),
                       dim3(kGqThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dsaidx
