// Cache write-back and current-chunk staging: token-major [tokens, H, D] in,
// head-major K rows and transposed V (V^T[h][d][key]) out (gfx950).
//
// A pure streaming kernel: each thread moves a P x P block (P = elements per 16
// bytes) of one head: P consecutive tokens times one 16-byte chunk of head_dim.
// It issues all of its loads first (K and V), writes the K pieces to their slot
// rows, transposes the V block in registers and writes P pieces of V^T rows.
// All accesses are 16 bytes wide; threads are ordered so that each store
// instruction covers whole 128-byte runs of a V^T row.  No LDS.
// [LB-fast] "3. KV 缓存 滚动窗口" / [ABot-stream] 机制二 (clean write-back of the
// chunk's K/V); the slot of each frame comes from the ring mapping on the host
// (FrameRun.dst0 = slot).
#include "skv_device.hpp"
#include "skv_kernels.hpp"

namespace skv {

namespace {

constexpr int kTT = 64;   // tokens per workgroup
constexpr int kThreads = 256;  // threads of the gather kernel

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

// Element e of each of the P 16-byte rows in, gathered into one 16-byte row: the
// transpose of a P x P block of 16- or 32-bit elements.
template <typename T>
__device__ __forceinline__ u32x4_t column(const u32x4_t (&in)[Per16<T>::n], int e) {
  u32x4_t r;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = (in[2 * w][e >> 1] >> (16 * (e & 1))) & 0xffffu;
      const uint32_t hi = (in[2 * w + 1][e >> 1] >> (16 * (e & 1))) & 0xffffu;
      r[w] = lo | (hi << 16);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) r[w] = in[w][e];
  }
  return r;
}

}  // namespace

// grid = (ceil(n_tok / 64) [or row_pad / 64 for staging], H); block = (64 / P) * (D / P) threads.
// Thread tid: token group tg = tid % (64 / P) (tokens t0 + P tg ...), chunk dc = tid / (64 / P).
template <typename T, int D>
__global__ __launch_bounds__(kTT / Per16<T>::n * (D / Per16<T>::n)) void write_kv_kernel(WriteArgs a) {
  constexpr int P = Per16<T>::n;  // elements per 16 bytes
  constexpr int NG = kTT / P;     // token groups per workgroup
  const int h = blockIdx.y;
  const int tg = threadIdx.x % NG, dc = threadIdx.x / NG;
  const int tb = blockIdx.x * kTT + tg * P;  // first token of this thread's block

  u32x4_t kv[P], vv[P];
  const u32x4_t z = {0u, 0u, 0u, 0u};
  // ---- every load first
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const bool ok = tb + j < a.n_tok;
    const int64_t off = (int64_t)(tb + j) * a.tok_stride + h * a.head_stride + dc * P;
    kv[j] = (a.k_src && ok) ? *(const u32x4_t*)((const T*)a.k_src + off) : z;
    vv[j] = ok ? *(const u32x4_t*)((const T*)a.v_src + off) : z;
  }
  // ---- K pieces -> head-major store rows (frame slot * F + token)
  if (a.k_src) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int gt = tb + j;
      if (gt < a.n_tok) {
        const int fi = gt / a.F, tok = gt - fi * a.F;
        const int64_t key = (int64_t)frame_dst(a, fi) * a.F + tok;
        *(u32x4_t*)((T*)a.k_dst + h * a.k_hs + key * D + dc * P) = kv[j];
      }
    }
  }
  // ---- V: P rows of V^T (d = dc * P + e), keys tb .. tb + P - 1
  T* vh = (T*)a.vt_dst + h * a.vt_hs;
  if (a.nruns == 0) {
    // staging: key = token; the row tail up to row_pad is written with the zeros loaded for it
    if (tb < a.row_pad) {
#pragma unroll
      for (int e = 0; e < P; ++e) *(u32x4_t*)(vh + (int64_t)(dc * P + e) * a.vt_ds + tb) = column<T>(vv, e);
    }
  } else if (tb < a.n_tok) {
    const int fi = tb / a.F, tok = tb - fi * a.F;
    const int64_t k0 = (int64_t)frame_dst(a, fi) * a.F + tok;
    const bool whole = tb + P <= a.n_tok && tok + P <= a.F && (k0 % P) == 0 && (a.vt_ds % P) == 0 &&
                       ((uintptr_t)vh & 15) == 0;
    if (whole) {
#pragma unroll
      for (int e = 0; e < P; ++e) *(u32x4_t*)(vh + (int64_t)(dc * P + e) * a.vt_ds + k0) = column<T>(vv, e);
    } else {
      for (int j = 0; j < P && tb + j < a.n_tok; ++j) {
        const int gt = tb + j, f2 = gt / a.F;
        const int64_t key = (int64_t)frame_dst(a, f2) * a.F + (gt - f2 * a.F);
        const T* src = (const T*)&vv[j];
#pragma unroll
        for (int e = 0; e < P; ++e) vh[(int64_t)(dc * P + e) * a.vt_ds + key] = src[e];
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
  constexpr int P = Per16<T>::n;
  switch (a.D) {
    case 32: hipLaunchKernelGGL((write_kv_kernel<T, 32>), grid, dim3(kTT / P * (32 / P)), 0, stream, a); break;
    case 64: hipLaunchKernelGGL((write_kv_kernel<T, 64>), grid, dim3(kTT / P * (64 / P)), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((write_kv_kernel<T, 128>), grid, dim3(kTT / P * (128 / P)), 0, stream, a); break;
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
