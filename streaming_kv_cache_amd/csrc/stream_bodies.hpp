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
  // the pair frequencies are loaded first, so that the angles wait only for them; the head loads
  // are unconditional (heads past the group's last load that one again) so none waits for another
  double om[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) om[p] = a.omega[g * 4 + p];
  const T* s = (const T*)j.src.base + (int64_t)(sf * a.F + tok) * j.src.tok_stride + g * 8 + h0 * j.src.head_stride;
  T* d = (T*)j.dst.base + (int64_t)(df * a.F + tok) * j.dst.tok_stride + g * 8 + h0 * j.dst.head_stride;
  typename IO::V x[kRopeHeads];
#pragma unroll
  for (int i = 0; i < kRopeHeads; ++i) x[i] = IO::load(s + (i < nh ? i : nh - 1) * j.src.head_stride);
  int64_t t = j.t0 + fi;
  if (j.clamp_max >= 0) t = t < 0 ? 0 : (t > j.clamp_max ? j.clamp_max : t);
  const int row = tok / a.gw, col = tok - row * a.gw;
  float cs[4], sn[4];
  const double two_pi = 6.283185307179586476925287;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int pair = g * 4 + p;
    const double pos = pair < a.pair_h ? (double)t : (pair < a.pair_w ? (double)row : (double)col);
    const double ang = pos * om[p];
    const double red = ang - two_pi * rint(ang / two_pi);  // |red| <= pi
    sincosf((float)red, &sn[p], &cs[p]);
  }
#pragma unroll
  for (int i = 0; i < kRopeHeads; ++i)
    if (i < nh) IO::rot_store(d + i * j.dst.head_stride, x[i], cs, sn);
}

// ---------------------------------------------------------------- K rows + V^T
// Cache write-back and current-chunk staging: token-major [tokens, H, D] in,
// head-major K rows and transposed V out (V^T in 64-key tiles for bf16, rows for fp32).
//
// A write block covers 64 consecutive keys of one head: staging keys (= tokens), or one
// 64-key tile of the key ranges the frames go to (write-back), so that a block whose keys
// all belong to the frames writes a whole, contiguous K block (64 rows) and, in bf16, a
// whole V^T tile.  Each thread moves a P x P block (P = elements per 16 bytes) of one head:
// P consecutive keys times one 16-byte chunk of head_dim.  It issues all of its loads first
// (K and V), writes the K pieces to their rows, transposes the V block in registers and
// writes P pieces of V^T.  All accesses are 16 bytes wide.
// [LB-fast] "3. KV 缓存 滚动窗口" / [ABot-stream] 机制二 (clean write-back of the
// chunk's K/V); the slot of each frame comes from the ring mapping on the host
// (FrameRun.dst0 = slot).
constexpr int kTT = kVtKeys;   // keys per write block

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

// V^T element (h's base vh, dim d, key j).
template <typename T>
__device__ __forceinline__ T* vt_elem(const WriteArgs& a, T* vh, int d, int64_t j) {
  return vh + (j / kTT) * a.vt_bs + (int64_t)d * a.vt_ds + j % kTT;
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

// One write block of write_block_threads<T, D>() threads: 64 keys of head h, block bx.
// Thread tid: key group tg = tid % (64 / P) (keys kb, kb + 1, ... kb + P - 1), chunk dc = tid / (64 / P).
// HAS_K: K rows are written too (else V only).  The common path is straight-line: every load
// (K, then V) is unconditional and issued before the first store, K rows are stored before the
// V^T pieces, so each group of stores waits only for its own loads.  A load under a lane
// condition, or a value merged across a branch, makes the compiler wait for loads (and for the
// stores issued before them) in between.
template <typename T, int D, bool HAS_K>
__device__ __forceinline__ void write_kv_block(const WriteArgs& a, unsigned bx, int h, unsigned tid) {
  constexpr int P = Per16<T>::n;  // elements per 16 bytes
  constexpr int NG = kTT / P;     // key groups per block
  const int tg = tid % NG, dc = tid / NG;
  // this block's keys, and the key range [klo, khi) of its frames with the token of key klo
  int kb, klo, khi, tok0;
  if (a.nruns == 0) {
    // staging: key = token; keys up to row_pad (tokens past n_tok are written as zeros)
    kb = (int)bx * kTT + tg * P;
    klo = 0;
    khi = a.row_pad;
    tok0 = 0;
  } else {
    // the run this block's tile belongs to (unrolled: no dynamic index into the arguments)
    int t0 = a.tile0[0], tp = a.tile_pre[0];
    FrameRun run = a.runs[0];
#pragma unroll
    for (int i = 1; i < 3; ++i)
      if (i < a.nruns && (int)bx >= a.tile_pre[i]) {
        t0 = a.tile0[i];
        tp = a.tile_pre[i];
        run = a.runs[i];
      }
    kb = (t0 + ((int)bx - tp)) * kTT + tg * P;
    klo = run.dst0 * a.F;
    khi = klo + run.count * a.F;
    tok0 = run.start * a.F;
  }
  if (kb + P <= klo || kb >= khi || a.n_tok <= 0) return;  // none of this thread's keys are written here
  T* vh = (T*)a.vt_dst + h * a.vt_hs;
  T* kh = HAS_K ? (T*)a.k_dst + h * a.k_hs : nullptr;
  if (kb >= klo && kb + P <= khi) {
    // P whole keys: tokens tb .. tb + P - 1; those past the last token (a staging block's padded
    // tail) load the last token and are zeroed by their mask
    const int tb = kb - klo + tok0, tl = a.n_tok - 1;
    const T* ks = HAS_K ? (const T*)a.k_src + h * a.head_stride + dc * P : nullptr;
    const T* vs = (const T*)a.v_src + h * a.head_stride + dc * P;
    u32x4_t kv[P], vv[P];
    if constexpr (HAS_K) {
#pragma unroll
      for (int j = 0; j < P; ++j) kv[j] = *(const u32x4_t*)(ks + (int64_t)(tb + j < tl ? tb + j : tl) * a.tok_stride);
    }
    // staging (V only) reads its source once and never again: nontemporal, so that it does not
    // displace the cache lines of the keys and values the attention pass reads next (pass
    // preparation at 480P -3.7 %; the write-back with K measured slower with it)
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const u32x4_t* src = (const u32x4_t*)(vs + (int64_t)(tb + j < tl ? tb + j : tl) * a.tok_stride);
      vv[j] = HAS_K ? *src : __builtin_nontemporal_load(src);
    }
    uint32_t m[P];
#pragma unroll
    for (int j = 0; j < P; ++j) m[j] = tb + j <= tl ? 0xffffffffu : 0u;
    if constexpr (HAS_K) {
      // ---- K pieces -> key rows
#pragma unroll
      for (int j = 0; j < P; ++j) {
        u32x4_t x = kv[j];
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] &= m[j];
        *(u32x4_t*)(kh + (int64_t)(kb + j) * D + dc * P) = x;
      }
    }
    // ---- V: P pieces of V^T (d = dc * P + e), keys kb .. kb + P - 1 (one 16-byte run: kb % P == 0)
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) vv[j][c] &= m[j];
#pragma unroll
    for (int e = 0; e < P; ++e) *(u32x4_t*)vt_elem<T>(a, vh, dc * P + e, kb) = column<T>(vv, e);
  } else {
    // a group cut by the frames' bounds (frames whose token count is not a multiple of P): key by key
    for (int j = 0; j < P; ++j) {
      const int key = kb + j;
      if (key < klo || key >= khi) continue;
      const int64_t off = (int64_t)(key - klo + tok0) * a.tok_stride + h * a.head_stride + dc * P;
      if (HAS_K) *(u32x4_t*)(kh + (int64_t)key * D + dc * P) = *(const u32x4_t*)((const T*)a.k_src + off);
      const u32x4_t v1 = *(const u32x4_t*)((const T*)a.v_src + off);
      const T* src = (const T*)&v1;
#pragma unroll
      for (int e = 0; e < P; ++e) *vt_elem<T>(a, vh, dc * P + e, key) = src[e];
    }
  }
}

}  // namespace skv
