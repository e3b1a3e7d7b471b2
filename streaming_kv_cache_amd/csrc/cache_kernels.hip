// Cache update, logical gather and 3D rotary kernels (gfx950).
//
// All three are HBM-bound streaming kernels.  Work is organised by token: a
// block owns a few tokens and its threads sweep the H*D elements of each token
// in 16-byte vectors, so every global access is a run of at least D*elt
// contiguous bytes on both the read and the write side, and index math per
// vector is a shift and a mask.
#include "skv_device.hpp"
#include "skv_kernels.hpp"

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
// [LB-src] 改造③ / [LB-causal] "Attention Sink" (start_frame offset) and
// [ABot-stream] 机制三 (relative ids over the visible window): token (frame i,
// row r, col w) turns pair k of the [time | height | width] part of head_dim by
// position * omega_k.  A block owns a few tokens and a group of kRopeHeads heads:
// each thread computes cos/sin for its 4 pairs once (angle reduced mod 2*pi in
// fp64, then fp32 sincos) and applies them to every head of the group, issuing
// all of its loads before the first store.
constexpr int kRopeThreads = 256;
constexpr int kRopeHeads = 8;

struct RopeArgs {
  RopeJob jobs[3];     // per grid z: tensors, time id of launch frame 0 (before clamping), clamp (>= 0)
  FrameRun runs[3];
  int32_t nruns;
  int32_t F, gw, H, D;
  int32_t pair_h, pair_w;  // first pair index of the height / width parts
  int32_t n_tok;
  double omega[64];    // per pair, theta^(-2k/d_axis) with k counted inside its axis
};

template <typename T>
struct RopeIo;

template <>
struct RopeIo<__bf16> {
  typedef u32x4_t V;  // 8 elements
  static __device__ __forceinline__ V load(const __bf16* p) { return *(const V*)p; }
  static __device__ __forceinline__ void rot_store(__bf16* d, const V& w, const float (&cs)[4], const float (&sn)[4]) {
    u32x4_t o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float x0 = bf16_lo_to_f32(w[p]), x1 = bf16_hi_to_f32(w[p]);
      o[p] = pack_bf16x2(x0 * cs[p] - x1 * sn[p], x0 * sn[p] + x1 * cs[p]);
    }
    *(u32x4_t*)d = o;
  }
};

template <>
struct RopeIo<float> {
  struct V {
    f32x4_t a, b;
  };
  static __device__ __forceinline__ V load(const float* p) { return V{*(const f32x4_t*)p, *(const f32x4_t*)(p + 4)}; }
  static __device__ __forceinline__ void rot_store(float* d, const V& v, const float (&cs)[4], const float (&sn)[4]) {
    const float x[8] = {v.a[0], v.a[1], v.a[2], v.a[3], v.b[0], v.b[1], v.b[2], v.b[3]};
    float y[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      y[2 * p] = x[2 * p] * cs[p] - x[2 * p + 1] * sn[p];
      y[2 * p + 1] = x[2 * p] * sn[p] + x[2 * p + 1] * cs[p];
    }
    *(f32x4_t*)d = f32x4_t{y[0], y[1], y[2], y[3]};
    *(f32x4_t*)(d + 4) = f32x4_t{y[4], y[5], y[6], y[7]};
  }
};

template <typename T>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(RopeArgs a) {
  using IO = RopeIo<T>;
  const int G = a.D >> 3;                 // groups of 4 pairs (8 elements) per row
  const int tpb = kRopeThreads / G;       // tokens per block
  const int g = threadIdx.x % G, tl = threadIdx.x / G;
  const int gt = blockIdx.x * tpb + tl;   // token index in the launch
  if (gt >= a.n_tok) return;
  const int h0 = blockIdx.y * kRopeHeads;
  const int nh = a.H - h0 < kRopeHeads ? a.H - h0 : kRopeHeads;
  const int fi = gt / a.F, tok = gt - fi * a.F;
  int sf = 0, df = 0;
  for (int r = 0; r < a.nruns; ++r) {
    const FrameRun run = a.runs[r];
    if (fi >= run.start && fi < run.start + run.count) {
      sf = run.src0 + (fi - run.start);
      df = run.dst0 + (fi - run.start);
    }
  }
  const RopeJob& j = a.jobs[blockIdx.z];
  const T* s = (const T*)j.src.base + (int64_t)(sf * a.F + tok) * j.src.tok_stride + g * 8 + h0 * j.src.head_stride;
  T* d = (T*)j.dst.base + (int64_t)(df * a.F + tok) * j.dst.tok_stride + g * 8 + h0 * j.dst.head_stride;
  typename IO::V x[kRopeHeads];
#pragma unroll
  for (int i = 0; i < kRopeHeads; ++i)
    if (i < nh) x[i] = IO::load(s + i * j.src.head_stride);
  int64_t t = j.t0 + fi;
  if (j.clamp_max >= 0) t = t < 0 ? 0 : (t > j.clamp_max ? j.clamp_max : t);
  const int row = tok / a.gw, col = tok - row * a.gw;
  float cs[4], sn[4];
  const double two_pi = 6.283185307179586476925287;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int pair = g * 4 + p;
    const double pos = pair < a.pair_h ? (double)t : (pair < a.pair_w ? (double)row : (double)col);
    const double ang = pos * a.omega[pair];
    const double red = ang - two_pi * rint(ang / two_pi);  // |red| <= pi
    sincosf((float)red, &sn[p], &cs[p]);
  }
#pragma unroll
  for (int i = 0; i < kRopeHeads; ++i)
    if (i < nh) IO::rot_store(d + i * j.dst.head_stride, x[i], cs, sn);
}

hipError_t launch_rope(const RopeLaunch& L, hipStream_t stream) {
  if (L.njobs < 1 || L.njobs > 3) return hipErrorInvalidValue;
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
  dim3 grid((a.n_tok + tpb - 1) / tpb, (L.H + kRopeHeads - 1) / kRopeHeads, L.njobs);
  if (L.dtype_bf16)
    hipLaunchKernelGGL(rope_kernel<__bf16>, grid, dim3(kRopeThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(kRopeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
