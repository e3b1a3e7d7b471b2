// Host-side bookkeeping of the streaming KV cache: configuration checks, the
// ring-slot state machine and the visible-set plan a chunk attends to.
//
// Pure C++17 with no HIP dependency, so the same code is compiled into the
// library and into a host-only test driver.
//
// Semantics ([LB-causal] "滑动窗口 KV 缓存" and "Attention Sink"; [LB-fast]
// "3. KV 缓存 滚动窗口"; [ABot-stream] 机制一):
//   * the logical cache is the first S frames ever appended (never evicted)
//     followed by the most recent (W - S) frames;
//   * a chunk of c frames sees every cached frame while cache + chunk fit in W,
//     else the sinks plus the most recent (W - S - c) frames, plus itself.
// Physically, frame f < S sits in slot f and frame f >= S in ring slot
// S + (f - S) mod (W - S): writing a frame into its ring slot overwrites exactly
// the oldest non-sink frame, which is the frame the pages' left shift drops.
#pragma once

#include <cstdint>
#include <cstddef>

#include "../../include/skv.h"

namespace skv {

struct Geometry {
  int32_t H = 0, D = 0, gh = 0, gw = 0, F = 0;
  int32_t c = 0, S = 0, W = 0, R = 0;   // R = W - S ring slots
  int32_t rope_t = 0, rope_h = 0, rope_w = 0;
  double theta = 10000.0;
  int32_t mode = SKV_ROPE_ABS;
  int32_t dtype = SKV_F32;
  int32_t elt = 4;                       // bytes per element
  int32_t fused = 0;                     // fused_rope: the library rotates q / k
};

// Check *cfg and fill the derived geometry (default split / theta applied).
skv_status make_geometry(const skv_config* cfg, Geometry* g);

// Head-dim support of the attention kernels for a dtype.
bool attention_head_dim_supported(int32_t dtype, int32_t D);

inline int64_t store_elems(const Geometry& g) { return (int64_t)g.W * g.F * g.H * g.D; }
// REL window keys rotated once per chunk (not used with fused rotation).
inline int64_t workspace_elems(const Geometry& g) {
  return g.mode == SKV_ROPE_REL && !g.fused ? (int64_t)(g.W - g.c) * g.F * g.H * g.D : 0;
}

// One contiguous run of visible history frames in physical slots, together with
// its place in the logical (oldest first) visible order.
struct SlotRun {
  int32_t slot0 = 0;     // first physical slot
  int32_t frames = 0;    // number of frames (consecutive slots)
  int32_t logical0 = 0;  // index of its first frame in the visible history
};

struct VisiblePlan {
  int32_t n_sink_vis = 0, n_ring_vis = 0, n_hist = 0, n_vis = 0;
  int32_t ring_start = -1;  // slot of the oldest visible ring frame
  int32_t n_runs = 0;       // <= 3 runs: sinks, ring part a, ring part b
  SlotRun runs[3];
  int64_t first_ring_frame = 0;  // frame id of the oldest visible ring frame
};

struct RingState {
  int64_t T = 0;  // frames appended so far

  int32_t slot_of(const Geometry& g, int64_t f) const {
    return f < g.S ? (int32_t)f : (int32_t)(g.S + (f - g.S) % g.R);
  }
  int32_t n_cached(const Geometry& g) const {
    int64_t sinks = T < g.S ? T : g.S;
    int64_t ring = T > g.S ? T - g.S : 0;
    if (ring > g.R) ring = g.R;
    return (int32_t)(sinks + ring);
  }
  // Frame id held at logical position i of the cache (0 = oldest).
  int64_t cached_frame(const Geometry& g, int32_t i) const {
    int32_t sinks = (int32_t)(T < g.S ? T : g.S);
    if (i < sinks) return i;
    int32_t ring = n_cached(g) - sinks;
    return T - ring + (i - sinks);
  }
  VisiblePlan plan(const Geometry& g, int32_t chunk) const;
};

}  // namespace skv
