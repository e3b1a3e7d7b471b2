// Cache write-back and current-chunk staging: token-major [tokens, H, D] in,
// head-major K rows and transposed V (V^T[h][d][key]) out (gfx950).
//
// One workgroup moves a tile of 64 tokens of one head: every thread issues all
// of its 16-byte loads (K and V) before any store, V goes through LDS to be
// transposed, and both outputs are written as runs of >= 128 contiguous bytes.
// The V store keeps V^T so that the attention kernel reads each 64-key tile of
// V^T as plain rows.  [LB-fast] "3. KV 缓存 滚动窗口" / [ABot-stream] 机制二
// (clean write-back of the chunk's K/V); the slot of each frame comes from the
// ring mapping on the host (FrameRun.dst0 = slot).
#include "skv_device.hpp"
#include "skv_kernels.hpp"

namespace skv {

namespace {

constexpr int kTT = 64;   // tokens per tile
constexpr int kThreads = 256;

template <typename T>
struct Per16 {
  static constexpr int n = 16 / sizeof(T);
};

// Frame position in key space (slot) of launch frame fi.
__device__ __forceinline__ int frame_dst(const WriteArgs& a, int fi) {
  int df = fi;
#pragma unroll
  for (int r = 0; r < 3; ++r)
    if (r < a.nruns && fi >= a.runs[r].start && fi < a.runs[r].start + a.runs[r].count)
      df = a.runs[r].dst0 + (fi - a.runs[r].start);
  return df;
}

}  // namespace

// grid = (ceil(n_tok / 64) [or row_pad / 64 for staging], H).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void write_kv_kernel(WriteArgs a) {
  constexpr int P = Per16<T>::n;           // elements per 16 bytes
  constexpr int VPR = D / P;               // 16-byte vectors per token row
  constexpr int NV = kTT * VPR / kThreads; // vectors per thread per tensor
  static_assert(NV * kThreads == kTT * VPR, "tile must split evenly");
  __shared__ T tile[kTT][D + P];           // V tile, padded rows
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * kTT;
  const int tid = threadIdx.x;

  u32x4_t kv[NV], vv[NV];
  const u32x4_t z = {0u, 0u, 0u, 0u};
  // ---- issue every load first
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = tid + i * kThreads;
    const int t = idx / VPR, c = idx % VPR;
    const bool ok = t0 + t < a.n_tok;
    const int64_t off = (int64_t)(t0 + t) * a.tok_stride + h * a.head_stride + c * P;
    kv[i] = (a.k_src && ok) ? *(const u32x4_t*)((const T*)a.k_src + off) : z;
    vv[i] = ok ? *(const u32x4_t*)((const T*)a.v_src + off) : z;
  }
  // ---- K rows -> head-major store rows (frame slot * F + token)
  if (a.k_src) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = tid + i * kThreads;
      const int t = idx / VPR, c = idx % VPR;
      const int gt = t0 + t;
      if (gt < a.n_tok) {
        const int fi = gt / a.F, tok = gt - fi * a.F;
        const int64_t key = (int64_t)frame_dst(a, fi) * a.F + tok;
        *(u32x4_t*)((T*)a.k_dst + h * a.k_hs + key * D + c * P) = kv[i];
      }
    }
  }
  // ---- V through LDS, written transposed
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = tid + i * kThreads;
    const int t = idx / VPR, c = idx % VPR;
    *(u32x4_t*)&tile[t][c * P] = vv[i];
  }
  __syncthreads();
  T* vh = (T*)a.vt_dst + h * a.vt_hs;
  constexpr int G = kTT / P;  // groups of P tokens per V^T row
#pragma unroll
  for (int i = 0; i < D * G / kThreads; ++i) {
    const int idx = tid + i * kThreads;
    const int d = idx / G, g = idx % G;
    const int tb = t0 + g * P;
    T* drow = vh + (int64_t)d * a.vt_ds;
    T vals[P];
#pragma unroll
    for (int e = 0; e < P; ++e) vals[e] = tile[g * P + e][d];
    if (a.nruns == 0) {
      // staging: key = token, row tail up to row_pad zero-filled (loads beyond n_tok gave zeros)
      if (tb < a.row_pad) *(u32x4_t*)(drow + tb) = __builtin_bit_cast(u32x4_t, vals);
    } else if (tb < a.n_tok) {
      const int fi = tb / a.F, tok = tb - fi * a.F;
      const int64_t k0 = (int64_t)frame_dst(a, fi) * a.F + tok;
      const bool whole = tb + P <= a.n_tok && tok + P <= a.F && (k0 % P) == 0 && ((uintptr_t)drow & 15) == 0;
      if (whole) {
        *(u32x4_t*)(drow + k0) = __builtin_bit_cast(u32x4_t, vals);
      } else {
        for (int e = 0; e < P && tb + e < a.n_tok; ++e) {
          const int gt = tb + e, f2 = gt / a.F;
          drow[(int64_t)frame_dst(a, f2) * a.F + (gt - f2 * a.F)] = vals[e];
        }
      }
    }
  }
}

// V^T -> token-major (logical gather, not on the hot path).  grid = (ceil(n_tok / 64), H);
// runs map launch frames to their slots.
template <typename T>
__global__ __launch_bounds__(kThreads) void vt_to_tok_kernel(WriteArgs a) {
  constexpr int P = Per16<T>::n;
  const int D = a.D;
  __shared__ T tile[kTT][128 + P];
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * kTT;
  const T* src = (const T*)a.vt_dst + h * a.vt_hs;
  T* dst = (T*)a.k_dst;  // token-major output
  for (int i = threadIdx.x; i < D * kTT; i += kThreads) {
    const int d = i / kTT, t = i - d * kTT;
    const int gt = t0 + t;
    if (gt < a.n_tok) {
      const int fi = gt / a.F;
      tile[t][d] = src[(int64_t)d * a.vt_ds + (int64_t)frame_dst(a, fi) * a.F + (gt - fi * a.F)];
    }
  }
  __syncthreads();
  const int vec_per_row = D / P;
  for (int i = threadIdx.x; i < kTT * vec_per_row; i += kThreads) {
    const int t = i / vec_per_row, c = i - t * vec_per_row;
    if (t0 + t < a.n_tok)
      *(u32x4_t*)(dst + (int64_t)(t0 + t) * a.tok_stride + h * a.head_stride + c * P) = *(const u32x4_t*)&tile[t][c * P];
  }
}

template <typename T>
static hipError_t launch_write_t(const WriteArgs& a, dim3 grid, hipStream_t stream) {
  switch (a.D) {
    case 32: hipLaunchKernelGGL((write_kv_kernel<T, 32>), grid, dim3(kThreads), 0, stream, a); break;
    case 64: hipLaunchKernelGGL((write_kv_kernel<T, 64>), grid, dim3(kThreads), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((write_kv_kernel<T, 128>), grid, dim3(kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_write_kv(const WriteArgs& a, int elt, hipStream_t stream) {
  dim3 grid((a.n_tok + kTT - 1) / kTT, a.H);
  if (a.nruns == 0) grid.x = (a.row_pad + kTT - 1) / kTT;
  return elt == 2 ? launch_write_t<uint16_t>(a, grid, stream) : launch_write_t<uint32_t>(a, grid, stream);
}

hipError_t launch_vt_to_tok(const WriteArgs& a, int elt, hipStream_t stream) {
  dim3 grid((a.n_tok + kTT - 1) / kTT, a.H);
  if (elt == 2)
    hipLaunchKernelGGL(vt_to_tok_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(vt_to_tok_kernel<uint32_t>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
