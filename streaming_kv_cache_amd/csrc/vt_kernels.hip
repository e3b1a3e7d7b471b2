// Token-major <-> transposed-V copies (gfx950).
//
// The V store keeps each head's values transposed, V^T[h][d][key], so that the
// attention kernel's second product reads V^T tiles as plain rows (keys are
// contiguous).  These kernels move whole frames between the caller's
// token-major [tokens, H, D] tensors and that layout through an LDS tile of 64
// tokens x D per head; both the global reads (token rows) and the global writes
// (runs of keys) are contiguous.
#include "skv_device.hpp"
#include "skv_kernels.hpp"

namespace skv {

namespace {

constexpr int kTT = 64;  // tokens per tile

template <typename T>
struct VtTraits;
template <>
struct VtTraits<uint16_t> {
  static constexpr int per16 = 8;
};
template <>
struct VtTraits<uint32_t> {
  static constexpr int per16 = 4;
};

// Key position in the V^T row space of the token gt of the launch.
__device__ __forceinline__ int64_t vt_key_of(const VtCopyArgs& a, int gt) {
  const int fi = gt / a.F, tok = gt - fi * a.F;
  int df = fi;
  for (int r = 0; r < a.nruns; ++r) {
    const FrameRun run = a.runs[r];
    if (fi >= run.start && fi < run.start + run.count) df = run.dst0 + (fi - run.start);
  }
  return (int64_t)df * a.F + tok;
}

}  // namespace

// Token-major -> V^T.  grid = (ceil(n_tok / 64), H).  Tokens of the launch are
// [0, n_tok); token gt of frame fi goes to key (slot of fi) * F + tok, or to key
// gt when there are no runs (the current-chunk workspace, whose row tail up to
// row_pad keys is zero-filled).
template <typename T>
__global__ __launch_bounds__(256) void tok_to_vt_kernel(VtCopyArgs a) {
  constexpr int P = VtTraits<T>::per16;     // elements per 16 bytes
  const int D = a.D;
  __shared__ T tile[kTT][128 + P];          // D <= 128
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * kTT;
  const T* src = (const T*)a.tok_base;
  T* dst = (T*)a.vt_base;
  // load 64 token rows of head h (16-byte vectors)
  const int vec_per_row = D / P;
  for (int i = threadIdx.x; i < kTT * vec_per_row; i += 256) {
    const int t = i / vec_per_row, c = i - t * vec_per_row;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (t0 + t < a.n_tok) v = *(const u32x4_t*)(src + (int64_t)(t0 + t) * a.tok_stride + h * a.head_stride + c * P);
    *(u32x4_t*)&tile[t][c * P] = v;
  }
  __syncthreads();
  // write D rows x 64 keys; groups of P consecutive tokens per thread
  const int groups = kTT / P;
  T* dh = dst + h * a.vt_hs;
  for (int i = threadIdx.x; i < D * groups; i += 256) {
    const int d = i / groups, g = i - d * groups;
    const int tb = g * P;
    T* drow = dh + (int64_t)d * a.vt_ds;
    if (a.nruns == 0) {
      // contiguous keys; the row is padded to a multiple of 64 keys and 16-byte aligned
      if (t0 + tb >= a.row_pad) continue;
      T vals[P];
#pragma unroll
      for (int e = 0; e < P; ++e) vals[e] = (t0 + tb + e < a.n_tok) ? tile[tb + e][d] : T(0);
      *(u32x4_t*)(drow + t0 + tb) = __builtin_bit_cast(u32x4_t, vals);
    } else {
      const int first = t0 + tb;
      if (first >= a.n_tok) continue;
      const int64_t k0 = vt_key_of(a, first);
      const bool whole = first + P <= a.n_tok && (k0 % P) == 0 && ((uintptr_t)drow & 15) == 0 &&
                         vt_key_of(a, first + P - 1) == k0 + P - 1;
      if (whole) {
        T vals[P];
#pragma unroll
        for (int e = 0; e < P; ++e) vals[e] = tile[tb + e][d];
        *(u32x4_t*)(drow + k0) = __builtin_bit_cast(u32x4_t, vals);
      } else {
        for (int e = 0; e < P && first + e < a.n_tok; ++e) drow[vt_key_of(a, first + e)] = tile[tb + e][d];
      }
    }
  }
}

// V^T -> token-major (logical gather).  grid = (ceil(n_tok / 64), H).  Runs map
// launch frames to their slots (source side).
template <typename T>
__global__ __launch_bounds__(256) void vt_to_tok_kernel(VtCopyArgs a) {
  constexpr int P = VtTraits<T>::per16;
  const int D = a.D;
  __shared__ T tile[kTT][128 + P];
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * kTT;
  const T* src = (const T*)a.vt_base + h * a.vt_hs;
  T* dst = (T*)a.tok_base;
  for (int i = threadIdx.x; i < D * kTT; i += 256) {
    const int d = i / kTT, t = i - d * kTT;
    if (t0 + t < a.n_tok) tile[t][d] = src[(int64_t)d * a.vt_ds + vt_key_of(a, t0 + t)];
  }
  __syncthreads();
  const int vec_per_row = D / P;
  for (int i = threadIdx.x; i < kTT * vec_per_row; i += 256) {
    const int t = i / vec_per_row, c = i - t * vec_per_row;
    if (t0 + t < a.n_tok)
      *(u32x4_t*)(dst + (int64_t)(t0 + t) * a.tok_stride + h * a.head_stride + c * P) = *(const u32x4_t*)&tile[t][c * P];
  }
}

hipError_t launch_tok_to_vt(const VtCopyArgs& a, int elt, hipStream_t stream) {
  dim3 grid((a.n_tok + kTT - 1) / kTT, a.H);
  if (a.nruns == 0) grid.x = (a.row_pad + kTT - 1) / kTT;  // also zero-fill the padded tail
  if (elt == 2)
    hipLaunchKernelGGL(tok_to_vt_kernel<uint16_t>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(tok_to_vt_kernel<uint32_t>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_vt_to_tok(const VtCopyArgs& a, int elt, hipStream_t stream) {
  dim3 grid((a.n_tok + kTT - 1) / kTT, a.H);
  if (elt == 2)
    hipLaunchKernelGGL(vt_to_tok_kernel<uint16_t>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(vt_to_tok_kernel<uint32_t>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
