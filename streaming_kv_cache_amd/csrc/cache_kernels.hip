// Frame copy (cache update of keys, logical gather), 3D rotary and pass
// preparation kernels (gfx950).
//
// All are HBM-bound streaming kernels.  Work is organised by token: a
// block owns a few tokens and its threads sweep the H*D elements of each token
// in 16-byte vectors, so every global access is a run of at least D*elt
// contiguous bytes on both the read and the write side, and index math per
// vector is a shift and a mask.
#include "stream_bodies.hpp"

namespace skv {

// ---------------------------------------------------------------- frame copy
// Copies whole frames between two token views, for up to two tensors at once
// (blockIdx.y selects the tensor).  Used for the keys by
//   * kv_cache_append_evict: caller's token-major chunk -> ring slots of the
//     head-major stores ([LB-fast] 3. KV 缓存 滚动窗口: write the clean chunk;
//     the ring slot of a frame is the one its evicted predecessor held), and
//   * kv_cache_gather: ring slots -> logical (oldest first) token-major copy.
constexpr int kCopyTokPerBlock = 4;
constexpr int kCopyThreads = 256;

struct CopyArgs {
  TokView src[2], dst[2];
  FrameRun runs[3];
  int32_t nruns;
  int32_t F, H, row_vec_shift;  // vectors per (token, head) row = 1 << row_vec_shift
  int32_t elt;
  int32_t n_tok;                // tokens in the launch
};

__global__ __launch_bounds__(kCopyThreads) void copy_frames_kernel(CopyArgs a) {
  const int which = blockIdx.y;
  const char* src = (const char*)a.src[which].base;
  char* dst = (char*)a.dst[which].base;
  const int64_t s_ts = a.src[which].tok_stride * a.elt, s_hs = a.src[which].head_stride * a.elt;
  const int64_t d_ts = a.dst[which].tok_stride * a.elt, d_hs = a.dst[which].head_stride * a.elt;
  const int row_vecs = 1 << a.row_vec_shift;
  const int per_tok = a.H << a.row_vec_shift;
  for (int tl = 0; tl < kCopyTokPerBlock; ++tl) {
    const int gt = blockIdx.x * kCopyTokPerBlock + tl;  // token index in the launch
    if (gt >= a.n_tok) break;
    const int fi = gt / a.F, tok = gt - fi * a.F;      // launch frame, token in frame
    int sf = 0, df = 0;
    for (int r = 0; r < a.nruns; ++r) {
      const FrameRun run = a.runs[r];
      if (fi >= run.start && fi < run.start + run.count) {
        sf = run.src0 + (fi - run.start);
        df = run.dst0 + (fi - run.start);
      }
    }
    const char* s_tok = src + (int64_t)(sf * a.F + tok) * s_ts;
    char* d_tok = dst + (int64_t)(df * a.F + tok) * d_ts;
    for (int t = threadIdx.x; t < per_tok; t += kCopyThreads) {
      const int h = t >> a.row_vec_shift, c = t & (row_vecs - 1);
      const u32x4_t v = *(const u32x4_t*)(s_tok + h * s_hs + c * 16);
      *(u32x4_t*)(d_tok + h * d_hs + c * 16) = v;
    }
  }
}

hipError_t launch_copy_frames(const TokView src[2], const TokView dst[2], int n_tensors, const FrameRun* runs,
                              int nruns, int n_frames, int F, int H, int D, int elt, hipStream_t stream) {
  CopyArgs a;
  for (int i = 0; i < 2; ++i) {
    a.src[i] = src[i];
    a.dst[i] = dst[i];
  }
  for (int i = 0; i < 3; ++i) a.runs[i] = i < nruns ? runs[i] : FrameRun{0, 0, 0, 0};
  a.nruns = nruns;
  a.F = F;
  a.H = H;
  int row_vecs = D * elt / 16, sh = 0;
  while ((1 << sh) < row_vecs) ++sh;
  a.row_vec_shift = sh;
  a.elt = elt;
  a.n_tok = n_frames * F;
  dim3 grid((a.n_tok + kCopyTokPerBlock - 1) / kCopyTokPerBlock, n_tensors);
  hipLaunchKernelGGL(copy_frames_kernel, grid, dim3(kCopyThreads), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- 3D RoPE
// Body and argument block in stream_bodies.hpp.  grid = (token blocks, head groups, tensors).
template <typename T>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(RopeArgs a) {
  rope_block<T>(a, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x);
}

// Fills the argument block of a rotary launch and its grid.
static RopeArgs rope_args(const RopeLaunch& L, dim3* grid) {
  RopeArgs a;
  for (int i = 0; i < 3; ++i) a.jobs[i] = L.job[i < L.njobs ? i : 0];
  for (int i = 0; i < 3; ++i) a.runs[i] = i < L.nruns ? L.runs[i] : FrameRun{0, 0, 0, 0};
  a.nruns = L.nruns;
  a.F = L.F;
  a.gw = L.gw;
  a.H = L.H;
  a.D = L.D;
  a.pair_h = L.rope_t / 2;
  a.pair_w = (L.rope_t + L.rope_h) / 2;
  a.n_tok = L.n_frames * L.F;
  // omega_k = theta^(-2k/d_axis), k counted from 0 inside each axis
  const int dims[3] = {L.rope_t, L.rope_h, L.rope_w};
  int p = 0;
  for (int ax = 0; ax < 3; ++ax)
    for (int k = 0; k < dims[ax] / 2; ++k) a.omega[p++] = pow(L.theta, -2.0 * k / (double)dims[ax]);
  for (; p < 64; ++p) a.omega[p] = 0.0;
  const int G = L.D / 8;
  const int tpb = kRopeThreads / G;
  *grid = dim3((a.n_tok + tpb - 1) / tpb, (L.H + kRopeHeads - 1) / kRopeHeads, L.njobs);
  return a;
}

hipError_t launch_rope(const RopeLaunch& L, hipStream_t stream) {
  if (L.njobs < 1 || L.njobs > 3) return hipErrorInvalidValue;
  dim3 grid;
  const RopeArgs a = rope_args(L, &grid);
  if (L.dtype_bf16)
    hipLaunchKernelGGL(rope_kernel<__bf16>, grid, dim3(kRopeThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(kRopeThreads), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- pass preparation
// The rotary blocks of a launch (q, k_cur, ...) and the blocks staging the chunk's V^T, in one
// bf16 grid: workgroups [0, n_rope) are rotary blocks in the rotary grid's order (x fastest),
// the rest carry kRopeThreads / write_block_threads() staging blocks each.  The two kinds read
// and write disjoint tensors, so their order within the grid does not matter; one launch saves
// the gap and the ramp of a second one before the attention pass.
template <int D>
__global__ __launch_bounds__(kRopeThreads) void prepare_pass_kernel(RopeArgs r, WriteArgs w, int rope_gx,
                                                                    int rope_gy, int n_rope, int stage_gx,
                                                                    int n_stage) {
  const int b = blockIdx.x;
  if (b < n_rope) {
    const int yz = b / rope_gx;
    rope_block<__bf16>(r, b - yz * rope_gx, yz % rope_gy, yz / rope_gy, threadIdx.x);
  } else {
    constexpr int WT = write_block_threads<uint16_t, D>();
    static_assert(kRopeThreads % WT == 0, "staging blocks must tile the workgroup");
    const int sb = (b - n_rope) * (kRopeThreads / WT) + (int)threadIdx.x / WT;
    if (sb >= n_stage) return;
    write_kv_block<uint16_t, D, false>(w, sb % stage_gx, sb / stage_gx, (int)threadIdx.x % WT);
  }
}

hipError_t launch_prepare_pass(const RopeLaunch& L, const WriteArgs& w, hipStream_t stream) {
  // the staging half writes V^T only (the rotary half writes k)
  if (L.njobs < 1 || L.njobs > 3 || !L.dtype_bf16 || w.nruns != 0 || w.k_src || L.D != w.D) return hipErrorInvalidValue;
  dim3 rg;
  const RopeArgs r = rope_args(L, &rg);
  const int n_rope = (int)(rg.x * rg.y * rg.z);
  const int stage_gx = (w.row_pad + kTT - 1) / kTT;
  const int n_stage = stage_gx * w.H;
  int per_wg;
  switch (w.D) {
    case 64: per_wg = kRopeThreads / write_block_threads<uint16_t, 64>(); break;
    case 128: per_wg = kRopeThreads / write_block_threads<uint16_t, 128>(); break;
    default: return hipErrorInvalidValue;
  }
  const dim3 grid(n_rope + (n_stage + per_wg - 1) / per_wg);
  switch (w.D) {
    case 64:
      hipLaunchKernelGGL(prepare_pass_kernel<64>, grid, dim3(kRopeThreads), 0, stream, r, w, (int)rg.x, (int)rg.y,
                         n_rope, stage_gx, n_stage);
      break;
    default:
      hipLaunchKernelGGL(prepare_pass_kernel<128>, grid, dim3(kRopeThreads), 0, stream, r, w, (int)rg.x, (int)rg.y,
                         n_rope, stage_gx, n_stage);
      break;
  }
  return hipGetLastError();
}

}  // namespace skv
