// Per-block bodies of the two streaming kernels that prepare an attention pass:
// the 3D rotary turn of token-major tensors and the write of K rows / V^T rows.
// Each kernel that runs them (rope_kernel, write_kv_kernel, and the combined
// preparation kernel that runs both kinds of block in one grid) passes the block
// coordinates in, so one source serves all of them.  Neither body uses LDS or a
// barrier: a block may leave early.
#pragma once

#include "skv_device.hpp"
#include "skv_kernels.hpp"

namespace skv {

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

// One rotary block of kRopeThreads threads: token block bx, head group by, tensor (job) bz.
template <typename T>
__device__ __forceinline__ void rope_block(const RopeArgs a, unsigned bx, unsigned by, unsigned bz, unsigned tid) {
  using IO = RopeIo<T>;
  const int G = a.D >> 3;                 // groups of 4 pairs (8 elements) per row
  const int tpb = kRopeThreads / G;       // tokens per block
  const int g = tid % G, tl = tid / G;
  const int gt = bx * tpb + tl;           // token index in the launch
  if (gt >= a.n_tok) return;
  const int h0 = by * kRopeHeads;
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
  const RopeJob& j = a.jobs[bz];
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

// ---------------------------------------------------------------- K rows + V^T
// Cache write-back and current-chunk staging: token-major [tokens, H, D] in,
// head-major K rows and transposed V (V^T[h][d][key]) out.
//
// Each thread moves a P x P block (P = elements per 16 bytes) of one head: P
// consecutive tokens times one 16-byte chunk of head_dim.  It issues all of its
// loads first (K and V), writes the K pieces to their slot rows, transposes the V
// block in registers and writes P pieces of V^T rows.  All accesses are 16 bytes
// wide; threads are ordered so that each store instruction covers whole 128-byte
// runs of a V^T row.
// [LB-fast] "3. KV 缓存 滚动窗口" / [ABot-stream] 机制二 (clean write-back of the
// chunk's K/V); the slot of each frame comes from the ring mapping on the host
// (FrameRun.dst0 = slot).
constexpr int kTT = 64;   // tokens per write block

template <typename T>
struct Per16 {
  static constexpr int n = 16 / sizeof(T);
};

// Threads of one write block.
template <typename T, int D>
constexpr int write_block_threads() {
  return kTT / Per16<T>::n * (D / Per16<T>::n);
}

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

// One write block of write_block_threads<T, D>() threads: tokens bx * 64 ... (+63) of head h
// (or, when staging, keys bx * 64 ... of the padded V^T rows).
// Thread tid: token group tg = tid % (64 / P) (tokens t0 + P tg ...), chunk dc = tid / (64 / P).
template <typename T, int D>
__device__ __forceinline__ void write_kv_block(const WriteArgs a, unsigned bx, int h, unsigned tid) {
  constexpr int P = Per16<T>::n;  // elements per 16 bytes
  constexpr int NG = kTT / P;     // token groups per block
  const int tg = tid % NG, dc = tid / NG;
  const int tb = bx * kTT + tg * P;  // first token of this thread's block

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

}  // namespace skv
