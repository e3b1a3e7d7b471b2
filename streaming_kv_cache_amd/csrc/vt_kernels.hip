// Cache write-back and current-chunk staging (K rows + transposed V, body in
// stream_bodies.hpp) and the V^T -> token-major gather (gfx950).
// [LB-fast] "3. KV 缓存 滚动窗口" / [ABot-stream] 机制二 (clean write-back of the
// chunk's K/V); the slot of each frame comes from the ring mapping on the host
// (FrameRun.dst0 = slot).
#include "stream_bodies.hpp"

namespace skv {

namespace {

constexpr int kThreads = 256;  // threads of the gather kernel

}  // namespace

// grid = (64-key tiles of the runs' keys [or row_pad / 64 for staging], H); block = write_block_threads<T, D>().
// HAS_K: K rows too (one instantiation each, so that the V-only one keeps its smaller register
// budget and occupancy).
template <typename T, int D, bool HAS_K>
__global__ __launch_bounds__((write_block_threads<T, D>())) void write_kv_kernel(WriteArgs a) {
  write_kv_block<T, D, HAS_K>(a, blockIdx.x, blockIdx.y, threadIdx.x);
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
      tile[t][d] = *vt_elem<const T>(a, src, d, (int64_t)frame_dst(a, fi) * a.F + (gt - fi * a.F));
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

template <typename T, bool HAS_K>
static hipError_t launch_write_t(const WriteArgs& a, dim3 grid, hipStream_t stream) {
  constexpr int P = Per16<T>::n;
  switch (a.D) {
    case 32: hipLaunchKernelGGL((write_kv_kernel<T, 32, HAS_K>), grid, dim3(kTT / P * (32 / P)), 0, stream, a); break;
    case 64: hipLaunchKernelGGL((write_kv_kernel<T, 64, HAS_K>), grid, dim3(kTT / P * (64 / P)), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((write_kv_kernel<T, 128, HAS_K>), grid, dim3(kTT / P * (128 / P)), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_write_kv(const WriteArgs& in, int elt, hipStream_t stream) {
  WriteArgs a = in;
  dim3 grid((a.row_pad + kTT - 1) / kTT, a.H);
  if (a.nruns > 0) {
    // one workgroup per 64-key tile touched by each run's keys [dst0 * F, (dst0 + count) * F)
    int total = 0;
    for (int r = 0; r < 3; ++r) {
      a.tile_pre[r] = total;
      a.tile0[r] = 0;
      if (r < a.nruns && a.runs[r].count > 0) {
        const int64_t lo = (int64_t)a.runs[r].dst0 * a.F, hi = lo + (int64_t)a.runs[r].count * a.F;
        a.tile0[r] = (int)(lo / kTT);
        total += (int)((hi - 1) / kTT - lo / kTT + 1);
      }
    }
    a.tile_pre[3] = total;
    grid.x = total;
  }
  if (grid.x == 0) return hipSuccess;
  if (a.k_src)
    return elt == 2 ? launch_write_t<uint16_t, true>(a, grid, stream) : launch_write_t<uint32_t, true>(a, grid, stream);
  return elt == 2 ? launch_write_t<uint16_t, false>(a, grid, stream) : launch_write_t<uint32_t, false>(a, grid, stream);
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
