// C ABI of the streaming KV cache (include/skv.h): argument checks, host-side
// ring bookkeeping and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <new>

#include "../../include/skv.h"
#include "skv_core.hpp"
#include "skv_kernels.hpp"

struct skv_cache {
  skv::Geometry g;
  skv::RingState ring;
  void* k_store = nullptr;
  void* v_store = nullptr;
  void* ws = nullptr;
  bool window_ready = false;
  bool v_staged = false;  // current-chunk values staged since the last append/reset
  bool poisoned = false;
};

namespace {

// Test hook (skv_debug_fail_launches): the next n launches report a failure without launching.
std::atomic<int32_t> g_fail_launches{0};

// Every kernel launch and device copy of the library goes through here.
template <class F>
hipError_t gate(F&& launch) {
  int32_t n = g_fail_launches.load();
  while (n > 0)
    if (g_fail_launches.compare_exchange_weak(n, n - 1)) return hipErrorLaunchFailure;
  return launch();
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

skv_status check_ptr(const void* p) {
  if (!p) return SKV_ERR_NULL;
  if (misaligned(p)) return SKV_ERR_ALIGN;
  return SKV_OK;
}

skv_status check_handle(const skv_cache* c) {
  if (!c) return SKV_ERR_NULL;
  if (c->poisoned) return SKV_ERR_STATE;
  return SKV_OK;
}

skv_status launched(skv_cache* c, hipError_t e) {
  if (e == hipSuccess) return SKV_OK;
  if (c) c->poisoned = true;
  return SKV_ERR_HIP;
}

const char* byte_ptr(const void* base, int64_t elems, int elt) { return (const char*)base + elems * elt; }

// Head-major store view: token t of slot-space, head h at (h*W*F + t)*D.
skv::TokView store_view(const skv::Geometry& g, void* base) {
  return skv::TokView{base, (int64_t)g.D, (int64_t)g.W * g.F * g.D};
}
// Caller's token-major [tokens, H, D] view.
skv::TokView token_view(const skv::Geometry& g, const void* base) {
  return skv::TokView{const_cast<void*>(base), (int64_t)g.H * g.D, (int64_t)g.D};
}

float softmax_scale_log2(int D) { return (float)(1.4426950408889634 / std::sqrt((double)D)); }

// V store: V^T of key = slot*F + token, W*F keys per head padded to whole 64-key tiles; bf16 in
// tiles ([h][key / 64][d][key % 64]), fp32 in rows ([h][d][key]).
int64_t vt_row(const skv::Geometry& g) { return ((int64_t)g.W * g.F + 63) / 64 * 64; }
// V^T strides of a buffer of `keys` keys per head (a multiple of 64) in the layout of g's dtype.
void set_vt(skv::WriteArgs& w, const skv::Geometry& g, int64_t keys) {
  w.vt_hs = (int64_t)g.D * keys;
  w.vt_bs = g.dtype == SKV_BF16 ? (int64_t)skv::kVtKeys * g.D : skv::kVtKeys;
  w.vt_ds = g.dtype == SKV_BF16 ? skv::kVtKeys : keys;
}
// Current-chunk V^T rows in the workspace: c*F keys padded to a multiple of 64.
int64_t cur_row(const skv::Geometry& g) { return ((int64_t)g.c * g.F + 63) / 64 * 64; }
// Workspace: [REL window keys, (W-c)*F*H*D (not with fused rotation)]
//            [fused rotation: q at absolute ids, q at slot ids (REL), k_cur at absolute ids; c*F*H*D each]
//            [current-chunk V^T, H*D*cur_row].
int64_t ws_window_elems(const skv::Geometry& g) { return skv::workspace_elems(g); }
int64_t chunk_elems(const skv::Geometry& g) { return (int64_t)g.c * g.F * g.H * g.D; }
int64_t ws_fused_elems(const skv::Geometry& g) {
  return g.fused ? chunk_elems(g) * (g.mode == SKV_ROPE_REL ? 3 : 2) : 0;
}
int64_t ws_total_elems(const skv::Geometry& g) {
  return ws_window_elems(g) + ws_fused_elems(g) + (int64_t)g.H * g.D * cur_row(g);
}
// Split keys (bf16, a chunk grid that fills less than half a dispatch round, e.g. few heads):
// up to split_cap partial results per query row after the other parts, at a 256-byte boundary:
// part_o [cap][c*F][H][D] fp32, then part_ml [cap][c*F][H][2] fp32.
int32_t split_cap(const skv::Geometry& g) {
  if (g.dtype != SKV_BF16) return 0;
  const int64_t wg4 = ((int64_t)g.c * g.F + 127) / 128 * g.H;  // 4-wave workgroups of one chunk
  if (2 * wg4 > 512) return 0;
  const int64_t cap = 512 / wg4;
  return (int32_t)(cap < 16 ? cap : 16);
}
int64_t ws_split_off(const skv::Geometry& g) { return (ws_total_elems(g) * g.elt + 255) / 256 * 256; }
int64_t ws_split_bytes(const skv::Geometry& g) {
  return (int64_t)split_cap(g) * g.c * g.F * g.H * (g.D + 2) * 4;
}
void* ws_q_abs(const skv_cache* c) { return (char*)c->ws + ws_window_elems(c->g) * c->g.elt; }
void* ws_k_cur(const skv_cache* c) { return (char*)ws_q_abs(c) + chunk_elems(c->g) * c->g.elt; }
void* ws_q_rel(const skv_cache* c) { return (char*)ws_k_cur(c) + chunk_elems(c->g) * c->g.elt; }
void* ws_vt(const skv_cache* c) { return (char*)c->ws + (ws_window_elems(c->g) + ws_fused_elems(c->g)) * c->g.elt; }

// Current chunk's V -> V^T rows in the workspace (tail zero-filled to a multiple of 64 keys).
skv::WriteArgs stage_args(const skv_cache* c, const void* v_cur) {
  const skv::Geometry& g = c->g;
  skv::WriteArgs wa{};
  wa.k_src = nullptr;
  wa.v_src = v_cur;
  wa.tok_stride = (int64_t)g.H * g.D;
  wa.head_stride = g.D;
  wa.vt_dst = ws_vt(c);
  set_vt(wa, g, cur_row(g));
  wa.nruns = 0;
  wa.F = g.F;
  wa.H = g.H;
  wa.D = g.D;
  wa.n_tok = g.c * g.F;
  wa.row_pad = (int32_t)cur_row(g);
  return wa;
}

skv_status stage_v(skv_cache* c, const void* v_cur, void* stream) {
  return launched(c, gate([&] { return skv::launch_write_kv(stage_args(c, v_cur), c->g.elt, (hipStream_t)stream); }));
}

// A rotary launch and the staging of v_cur: one grid in bf16, two launches in fp32.
skv_status rope_and_stage(skv_cache* c, const skv::RopeLaunch& L, const void* v_cur, void* stream) {
  const skv::WriteArgs w = stage_args(c, v_cur);
  if (c->g.dtype == SKV_BF16)
    return launched(c, gate([&] { return skv::launch_prepare_pass(L, w, (hipStream_t)stream); }));
  const skv_status st = launched(c, gate([&] { return skv::launch_rope(L, (hipStream_t)stream); }));
  if (st != SKV_OK) return st;
  return launched(c, gate([&] { return skv::launch_write_kv(w, c->g.elt, (hipStream_t)stream); }));
}

// Rotary launch over n_frames frames of a token-major tensor (or the store, via runs).
skv::RopeLaunch rope_launch(const skv::Geometry& g, skv::TokView src, skv::TokView dst, int32_t n_frames,
                            int64_t t0, int64_t clamp_max) {
  skv::RopeLaunch L;
  L.job[0] = skv::RopeJob{src, dst, t0, (int32_t)clamp_max};
  L.job[1] = L.job[2] = L.job[0];
  L.njobs = 1;
  L.runs[0] = skv::FrameRun{0, n_frames, 0, 0};
  L.nruns = 1;
  L.n_frames = n_frames;
  L.F = g.F;
  L.gw = g.gw;
  L.H = g.H;
  L.D = g.D;
  L.rope_t = g.rope_t;
  L.rope_h = g.rope_h;
  L.rope_w = g.rope_w;
  L.theta = g.theta;
  L.dtype_bf16 = g.dtype == SKV_BF16;
  return L;
}

// Fused rotation before an attention pass, into the workspace, in one launch: job 0 q at absolute
// ids, job 1 k_cur at absolute ids, job 2 (REL with visible sinks) q at slot ids.
skv::RopeLaunch fused_rope_launch(const skv_cache* c, const void* q, const void* k_cur) {
  const skv::Geometry& g = c->g;
  const skv::VisiblePlan p = c->ring.plan(g, g.c);
  const int64_t T = c->ring.T;
  skv::RopeLaunch L = rope_launch(g, token_view(g, q), token_view(g, ws_q_abs(c)), g.c, T, -1);
  L.job[1] = skv::RopeJob{token_view(g, k_cur), token_view(g, ws_k_cur(c)), T, -1};
  L.njobs = 2;
  if (g.mode == SKV_ROPE_REL && p.n_sink_vis > 0)
    L.job[L.njobs++] = skv::RopeJob{token_view(g, q), token_view(g, ws_q_rel(c)), p.n_vis - g.c, g.W - 1};
  return L;
}

}  // namespace

extern "C" {

skv_status kv_cache_stage_v(skv_cache* c, const void* v_cur, int32_t n_frames, void* stream) {
  skv_status st = check_handle(c);
  if (st != SKV_OK) return st;
  if ((st = check_ptr(v_cur)) != SKV_OK) return st;
  if (n_frames != c->g.c) return SKV_ERR_SHAPE;
  st = stage_v(c, v_cur, stream);
  if (st == SKV_OK) c->v_staged = true;
  return st;
}


int skv_abi_version(void) { return SKV_ABI_VERSION; }

const char* skv_status_string(skv_status s) {
  switch (s) {
    case SKV_OK: return "ok";
    case SKV_ERR_NULL: return "null pointer";
    case SKV_ERR_CONFIG: return "invalid or unsupported configuration";
    case SKV_ERR_SHAPE: return "frame or token count out of range";
    case SKV_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case SKV_ERR_STATE: return "call not valid in the cache's state (or cache poisoned by a failed launch)";
    case SKV_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

skv_status kv_cache_bytes(const skv_config* cfg, size_t* store_bytes_each, size_t* workspace_bytes) {
  if (!cfg || !store_bytes_each || !workspace_bytes) return SKV_ERR_NULL;
  skv::Geometry g;
  skv_status st = skv::make_geometry(cfg, &g);
  if (st != SKV_OK) return st;
  // the V store (V^T padded to whole 64-key tiles) is at least the K store's W*F*H*D elements
  *store_bytes_each = (size_t)(g.H * g.D * vt_row(g)) * g.elt;
  *workspace_bytes = (size_t)(ws_split_off(g) + ws_split_bytes(g));
  return SKV_OK;
}

skv_status kv_cache_init(const skv_config* cfg, void* k_store, void* v_store, void* workspace, skv_cache** out) {
  if (!cfg || !out) return SKV_ERR_NULL;
  skv::Geometry g;
  skv_status st = skv::make_geometry(cfg, &g);
  if (st != SKV_OK) return st;
  if ((st = check_ptr(k_store)) != SKV_OK) return st;
  if ((st = check_ptr(v_store)) != SKV_OK) return st;
  if ((st = check_ptr(workspace)) != SKV_OK) return st;
  skv_cache* c = new (std::nothrow) skv_cache();
  if (!c) return SKV_ERR_STATE;
  c->g = g;
  c->k_store = k_store;
  c->v_store = v_store;
  c->ws = workspace;
  *out = c;
  return SKV_OK;
}

skv_status kv_cache_reset(skv_cache* c) {
  if (!c) return SKV_ERR_NULL;
  c->ring.T = 0;
  c->window_ready = false;
  c->v_staged = false;
  c->poisoned = false;
  return SKV_OK;
}

skv_status kv_cache_destroy(skv_cache* c) {
  delete c;
  return SKV_OK;
}

skv_status kv_cache_info(const skv_cache* c, kv_cache_info_t* info) {
  if (!c || !info) return SKV_ERR_NULL;
  const skv::VisiblePlan p = c->ring.plan(c->g, c->g.c);
  info->n_appended = c->ring.T;
  info->n_cached = c->ring.n_cached(c->g);
  info->n_sink_vis = p.n_sink_vis;
  info->n_ring_vis = p.n_ring_vis;
  info->n_vis = p.n_vis;
  info->ring_start = p.ring_start;
  info->window_ready = c->window_ready ? 1 : 0;
  info->poisoned = c->poisoned ? 1 : 0;
  return SKV_OK;
}

skv_status kv_cache_append_evict(skv_cache* c, const void* k, const void* v, int32_t n_frames, void* stream) {
  skv_status st = check_handle(c);
  if (st != SKV_OK) return st;
  if ((st = check_ptr(k)) != SKV_OK) return st;
  if ((st = check_ptr(v)) != SKV_OK) return st;
  const skv::Geometry& g = c->g;
  if (n_frames < 1 || n_frames > g.W - g.S) return SKV_ERR_SHAPE;
  // frames T .. T+n-1 -> their slots, merged into runs of consecutive slots
  skv::FrameRun runs[3];
  int nruns = 0;
  for (int i = 0; i < n_frames; ++i) {
    const int slot = c->ring.slot_of(g, c->ring.T + i);
    if (nruns > 0 && runs[nruns - 1].dst0 + runs[nruns - 1].count == slot) {
      ++runs[nruns - 1].count;
    } else {
      if (nruns == 3) return SKV_ERR_STATE;  // cannot happen for n <= W - S
      runs[nruns++] = skv::FrameRun{i, 1, i, slot};
    }
  }
  if (g.fused) {
    // k rotated at the frames' absolute ids straight into their slots; V below
    skv::RopeLaunch L = rope_launch(g, token_view(g, k), store_view(g, c->k_store), n_frames, c->ring.T, -1);
    L.nruns = nruns;
    for (int i = 0; i < 3; ++i) L.runs[i] = i < nruns ? runs[i] : skv::FrameRun{0, 0, 0, 0};
    st = launched(c, gate([&] { return skv::launch_rope(L, (hipStream_t)stream); }));
    if (st != SKV_OK) return st;
  }
  skv::WriteArgs wa{};
  wa.k_src = g.fused ? nullptr : k;
  wa.v_src = v;
  wa.tok_stride = (int64_t)g.H * g.D;
  wa.head_stride = g.D;
  wa.k_dst = c->k_store;
  wa.k_hs = (int64_t)g.W * g.F * g.D;
  wa.vt_dst = c->v_store;
  set_vt(wa, g, vt_row(g));
  for (int i = 0; i < 3; ++i) wa.runs[i] = i < nruns ? runs[i] : skv::FrameRun{0, 0, 0, 0};
  wa.nruns = nruns;
  wa.F = g.F;
  wa.H = g.H;
  wa.D = g.D;
  wa.n_tok = n_frames * g.F;
  wa.row_pad = 0;
  st = launched(c, gate([&] { return skv::launch_write_kv(wa, g.elt, (hipStream_t)stream); }));
  if (st != SKV_OK) return st;
  c->ring.T += n_frames;
  c->window_ready = false;
  c->v_staged = false;
  return SKV_OK;
}

// rope_apply / rope_apply_qk / kv_cache_prepare_pass: checks n (1 or 2) tensors and describes one
// rotary launch over them with the same time ids; enqueues nothing.
static skv_status rope_plan(const skv_cache* c, const void* const* in, void* const* out, int n, int32_t n_frames,
                            int64_t start_frame, skv::RopeLaunch* L) {
  skv_status st = check_handle(c);
  if (st != SKV_OK) return st;
  for (int i = 0; i < n; ++i) {
    if ((st = check_ptr(in[i])) != SKV_OK) return st;
    if ((st = check_ptr(out[i])) != SKV_OK) return st;
  }
  const skv::Geometry& g = c->g;
  if (n_frames < 1 || (int64_t)n_frames * g.F > (int64_t)INT32_MAX / 2) return SKV_ERR_SHAPE;
  int64_t t0;
  int32_t clamp_max;
  if (g.mode == SKV_ROPE_ABS) {
    if (start_frame < 0) return SKV_ERR_SHAPE;
    t0 = start_frame;
    clamp_max = -1;
  } else {
    if (n_frames != g.c) return SKV_ERR_SHAPE;
    const skv::VisiblePlan p = c->ring.plan(g, g.c);
    t0 = p.n_vis - g.c;
    clamp_max = g.W - 1;
  }
  *L = rope_launch(g, token_view(g, in[0]), token_view(g, out[0]), n_frames, t0, clamp_max);
  for (int i = 1; i < n; ++i) L->job[i] = skv::RopeJob{token_view(g, in[i]), token_view(g, out[i]), t0, clamp_max};
  L->njobs = n;
  return SKV_OK;
}

static skv_status rope_tensors(const skv_cache* cc, const void* const* in, void* const* out, int n, int32_t n_frames,
                               int64_t start_frame, void* stream) {
  skv_cache* c = const_cast<skv_cache*>(cc);
  skv::RopeLaunch L;
  const skv_status st = rope_plan(c, in, out, n, n_frames, start_frame, &L);
  if (st != SKV_OK) return st;
  return launched(c, gate([&] { return skv::launch_rope(L, (hipStream_t)stream); }));
}

skv_status rope_apply(const skv_cache* cache, const void* x_in, void* x_out, int32_t n_frames, int64_t start_frame,
                      void* stream) {
  const void* in[1] = {x_in};
  void* out[1] = {x_out};
  return rope_tensors(cache, in, out, 1, n_frames, start_frame, stream);
}

skv_status rope_apply_qk(const skv_cache* cache, const void* q_in, void* q_out, const void* k_in, void* k_out,
                         int32_t n_frames, int64_t start_frame, void* stream) {
  const void* in[2] = {q_in, k_in};
  void* out[2] = {q_out, k_out};
  return rope_tensors(cache, in, out, 2, n_frames, start_frame, stream);
}

skv_status kv_cache_prepare_pass(skv_cache* c, const void* q_in, void* q_out, const void* k_in, void* k_out,
                                 const void* v_cur, int32_t n_frames, int64_t start_frame, void* stream) {
  const void* in[2] = {q_in, k_in};
  void* out[2] = {q_out, k_out};
  skv::RopeLaunch L;
  skv_status st = rope_plan(c, in, out, 2, n_frames, start_frame, &L);
  if (st != SKV_OK) return st;
  if ((st = check_ptr(v_cur)) != SKV_OK) return st;
  if (n_frames != c->g.c) return SKV_ERR_SHAPE;
  if (c->g.fused) return SKV_ERR_STATE;  // chunk_attention rotates (and stages) itself
  st = rope_and_stage(c, L, v_cur, stream);
  if (st == SKV_OK) c->v_staged = true;
  return st;
}

skv_status rope_apply_window(skv_cache* c, void* stream) {
  skv_status st = check_handle(c);
  if (st != SKV_OK) return st;
  const skv::Geometry& g = c->g;
  if (g.mode != SKV_ROPE_REL || g.fused) return SKV_ERR_STATE;
  const skv::VisiblePlan p = c->ring.plan(g, g.c);
  if (p.n_hist > 0) {
    skv::RopeLaunch L = rope_launch(g, store_view(g, c->k_store),
                                    skv::TokView{c->ws, (int64_t)g.D, (int64_t)(g.W - g.c) * g.F * g.D}, p.n_hist,
                                    0, g.W - 1);
    L.nruns = p.n_runs;
    for (int i = 0; i < p.n_runs; ++i)
      L.runs[i] = skv::FrameRun{p.runs[i].logical0, p.runs[i].frames, p.runs[i].slot0, p.runs[i].logical0};
    st = launched(c, gate([&] { return skv::launch_rope(L, (hipStream_t)stream); }));
    if (st != SKV_OK) return st;
  }
  c->window_ready = true;
  return SKV_OK;
}

// Checks one chunk_attention call and describes its key ranges; enqueues nothing.
static skv_status attention_args(skv_cache* c, const void* q, const void* k_cur, const void* v_cur, int32_t n_frames,
                                 void* out, skv::AttnArgs* a) {
  skv_status st = check_handle(c);
  if (st != SKV_OK) return st;
  if ((st = check_ptr(q)) != SKV_OK) return st;
  if ((st = check_ptr(k_cur)) != SKV_OK) return st;
  if (v_cur && misaligned(v_cur)) return SKV_ERR_ALIGN;
  if ((st = check_ptr(out)) != SKV_OK) return st;
  const skv::Geometry& g = c->g;
  if (n_frames != g.c) return SKV_ERR_SHAPE;
  const skv::VisiblePlan p = c->ring.plan(g, g.c);
  const bool rel = g.mode == SKV_ROPE_REL;
  if (rel && !g.fused && p.n_hist > 0 && !c->window_ready) return SKV_ERR_STATE;
  if (!v_cur && !c->v_staged) return SKV_ERR_STATE;

  // fused rotation: the workspace copies written by the fused rotary launch; REL sinks use the queries at
  // slot ids, everything after them the queries at absolute ids
  a->q = q;
  a->q_alt = nullptr;
  a->alt_seg = 1 << 20;
  if (g.fused) {
    const bool rel_sinks = rel && p.n_sink_vis > 0;
    a->q = rel_sinks ? ws_q_rel(c) : ws_q_abs(c);
    a->q_alt = ws_q_abs(c);
    a->alt_seg = rel_sinks ? 1 : 1 << 20;
    k_cur = ws_k_cur(c);
  }
  a->out = out;
  a->Lq = g.c * g.F;
  a->H = g.H;
  a->sl2 = softmax_scale_log2(g.D);
  a->nseg = 0;
  a->split_cap = split_cap(g);
  if (a->split_cap > 1) {
    char* base = (char*)c->ws + ws_split_off(g);
    a->part_o = (float*)base;
    a->part_ml = (float*)(base + (int64_t)a->split_cap * g.c * g.F * g.H * g.D * 4);
  }
  const int64_t store_hs = (int64_t)g.W * g.F * g.D;
  const int64_t ws_hs = (int64_t)(g.W - g.c) * g.F * g.D;
  const int per16 = 16 / g.elt;
  for (int i = 0; i < p.n_runs; ++i) {
    const skv::SlotRun& r = p.runs[i];
    skv::KvSeg sg;
    if (rel && !g.fused) {
      sg.k = byte_ptr(c->ws, (int64_t)r.logical0 * g.F * g.D, g.elt);
      sg.k_hs = ws_hs;
    } else {
      sg.k = byte_ptr(c->k_store, (int64_t)r.slot0 * g.F * g.D, g.elt);
      sg.k_hs = store_hs;
    }
    sg.k_rs = g.D;
    const int64_t key0 = (int64_t)r.slot0 * g.F;
    sg.v_hs = (int64_t)g.D * vt_row(g);
    sg.v_rs = 1;
    if (g.dtype == SKV_BF16) {
      // the tile holding key0; key0 sits at position key0 % 64 of it
      sg.v = byte_ptr(c->v_store, key0 / skv::kVtKeys * skv::kVtKeys * g.D, g.elt);
      sg.v_phase = (int32_t)(key0 % skv::kVtKeys);
      sg.v_ds = skv::kVtKeys;
    } else {
      sg.v = byte_ptr(c->v_store, key0, g.elt);
      sg.v_phase = 0;
      sg.v_ds = vt_row(g);
    }
    sg.n = r.frames * g.F;
    // 16-byte pieces of 8 keys: the range must start and end on a piece boundary, since the last
    // piece of a partial tile is read whole and the keys after the range may never have been written
    sg.v_al16 = (key0 % per16 == 0 && sg.n % per16 == 0) ? 1 : 0;
    a->seg[a->nseg++] = sg;
  }
  skv::KvSeg cur;
  cur.k = k_cur;
  cur.k_hs = g.D;
  cur.k_rs = (int64_t)g.H * g.D;
  cur.v = ws_vt(c);
  cur.v_hs = (int64_t)g.D * cur_row(g);
  cur.v_rs = 1;
  cur.v_ds = g.dtype == SKV_BF16 ? skv::kVtKeys : cur_row(g);
  cur.n = g.c * g.F;
  cur.v_al16 = 1;
  cur.v_phase = 0;
  a->seg[a->nseg++] = cur;
  for (int i = a->nseg; i < 4; ++i) a->seg[i] = skv::KvSeg{nullptr, nullptr, 0, 0, 0, 0, 0, 0, 0, 0};
  return SKV_OK;
}

static bool same_geometry(const skv::Geometry& x, const skv::Geometry& y) {
  return x.H == y.H && x.D == y.D && x.gh == y.gh && x.gw == y.gw && x.c == y.c && x.S == y.S && x.W == y.W &&
         x.dtype == y.dtype && x.mode == y.mode && x.fused == y.fused;
}

skv_status chunk_attention_batch(const skv_cache* const* caches, int32_t n_caches, const void* const* q,
                                 const void* const* k_cur, const void* const* v_cur, int32_t n_frames,
                                 void* const* out, void* stream) {
  if (!caches || !q || !k_cur || !out) return SKV_ERR_NULL;
  if (n_caches < 1 || n_caches > skv::kMaxAttnBatch) return SKV_ERR_SHAPE;
  skv::AttnBatch ab{};
  ab.nb = n_caches;
  skv_cache* cs[skv::kMaxAttnBatch];
  for (int i = 0; i < n_caches; ++i) {
    cs[i] = const_cast<skv_cache*>(caches[i]);
    if (!cs[i]) return SKV_ERR_NULL;
    for (int j = 0; j < i; ++j)
      if (cs[j] == cs[i]) return SKV_ERR_STATE;  // one handle twice: its staged values would clash
    const skv_status st = attention_args(cs[i], q[i], k_cur[i], v_cur ? v_cur[i] : nullptr, n_frames, out[i],
                                         &ab.b[i]);
    if (st != SKV_OK) return st;
    if (!same_geometry(cs[i]->g, cs[0]->g)) return SKV_ERR_CONFIG;
  }
  // everything checked: rotate (fused), stage the values given, then one launch for all elements
  for (int i = 0; i < n_caches; ++i) {
    const bool stage = v_cur && v_cur[i];
    skv_status st = SKV_OK;
    if (cs[i]->g.fused) {
      const skv::RopeLaunch L = fused_rope_launch(cs[i], q[i], k_cur[i]);
      st = stage ? rope_and_stage(cs[i], L, v_cur[i], stream)
                 : launched(cs[i], gate([&] { return skv::launch_rope(L, (hipStream_t)stream); }));
    } else if (stage) {
      st = stage_v(cs[i], v_cur[i], stream);
    }
    if (st != SKV_OK) return st;
    if (stage) cs[i]->v_staged = true;
  }
  const skv::Geometry& g = cs[0]->g;
  hipError_t e = hipSuccess;
  if (g.dtype == SKV_BF16) {
    e = gate([&] { return skv::launch_attention_bf16_vt(ab, g.D, (hipStream_t)stream); });
  } else {
    for (int i = 0; i < n_caches && e == hipSuccess; ++i)
      e = gate([&] { return skv::launch_attention_f32(ab.b[i], g.D, (hipStream_t)stream); });
  }
  skv_status st = SKV_OK;
  for (int i = 0; i < n_caches; ++i) {
    const skv_status si = launched(cs[i], e);
    if (si != SKV_OK) st = si;
  }
  return st;
}

skv_status chunk_attention(const skv_cache* cc, const void* q, const void* k_cur, const void* v_cur,
                           int32_t n_frames, void* out, void* stream) {
  return chunk_attention_batch(&cc, 1, &q, &k_cur, &v_cur, n_frames, &out, stream);
}

skv_status cross_attention(const void* q, int32_t n_q, const void* k_text, const void* v_text, int32_t n_text,
                           int32_t heads, int32_t head_dim, int32_t dtype, void* out, void* stream) {
  skv_status st;
  if ((st = check_ptr(q)) != SKV_OK) return st;
  if ((st = check_ptr(k_text)) != SKV_OK) return st;
  if ((st = check_ptr(v_text)) != SKV_OK) return st;
  if ((st = check_ptr(out)) != SKV_OK) return st;
  if (heads < 1 || heads > 4096) return SKV_ERR_CONFIG;
  if (!skv::attention_head_dim_supported(dtype, head_dim)) return SKV_ERR_CONFIG;
  if (n_q < 1 || n_text < 1 || (int64_t)n_text > (int64_t)INT32_MAX / 2 ||
      (int64_t)n_q * heads > (int64_t)INT32_MAX / 2)
    return SKV_ERR_SHAPE;
  skv::AttnArgs a{};
  a.q = q;
  a.out = out;
  a.alt_seg = 1 << 20;
  a.Lq = n_q;
  a.H = heads;
  a.sl2 = softmax_scale_log2(head_dim);
  a.nseg = 1;
  a.seg[0] = skv::KvSeg{k_text, v_text, (int64_t)head_dim, (int64_t)heads * head_dim,
                        (int64_t)head_dim, (int64_t)heads * head_dim, 1, n_text, 0};
  for (int i = 1; i < 4; ++i) a.seg[i] = skv::KvSeg{nullptr, nullptr, 0, 0, 0, 0, 0, 0, 0, 0};
  const hipError_t e = dtype == SKV_BF16 ? gate([&] { return skv::launch_attention_bf16_tokv(a, head_dim, (hipStream_t)stream); })
                                         : gate([&] { return skv::launch_attention_f32(a, head_dim, (hipStream_t)stream); });
  return e == hipSuccess ? SKV_OK : SKV_ERR_HIP;
}

// Prepared text cache: bf16 [K head-major, H*pad*D] [256-byte boundary] [V^T tiles, H*D*pad];
// fp32 [copy of k_text, n_text*H*D] [256-byte boundary] [copy of v_text].
struct TextLayout {
  int64_t k_bytes = 0, vt_off = 0, total = 0, pad = 0;
};

static skv_status text_layout(int32_t n_text, int32_t heads, int32_t head_dim, int32_t dtype, TextLayout* L) {
  if (heads < 1 || heads > 4096) return SKV_ERR_CONFIG;
  if (!skv::attention_head_dim_supported(dtype, head_dim)) return SKV_ERR_CONFIG;
  if (n_text < 1 || n_text > (1 << 30)) return SKV_ERR_SHAPE;
  const int64_t elt = dtype == SKV_BF16 ? 2 : 4;
  L->pad = ((int64_t)n_text + 63) / 64 * 64;
  // bf16: one head's keys are contiguous rows (as in the K store), padded with zero rows
  L->k_bytes = dtype == SKV_BF16 ? (int64_t)heads * L->pad * head_dim * 2 : (int64_t)n_text * heads * head_dim * elt;
  L->vt_off = (L->k_bytes + 255) / 256 * 256;
  if (dtype == SKV_BF16) {
    // the matrix-core kernel addresses one head's keys and V^T with 32-bit byte offsets
    if ((int64_t)head_dim * L->pad * 2 > INT32_MAX) return SKV_ERR_SHAPE;
    L->total = L->vt_off + (int64_t)heads * head_dim * L->pad * 2;
  } else {
    L->total = L->vt_off + L->k_bytes;
  }
  return SKV_OK;
}

static skv_status check_store(const void* store) {
  if (!store) return SKV_ERR_NULL;
  return ((uintptr_t)store & 255) ? SKV_ERR_ALIGN : SKV_OK;
}

skv_status text_cache_bytes(int32_t n_text, int32_t heads, int32_t head_dim, int32_t dtype, size_t* bytes) {
  if (!bytes) return SKV_ERR_NULL;
  TextLayout L;
  const skv_status st = text_layout(n_text, heads, head_dim, dtype, &L);
  if (st != SKV_OK) return st;
  *bytes = (size_t)L.total;
  return SKV_OK;
}

skv_status text_cache_prepare(const void* k_text, const void* v_text, int32_t n_text, int32_t heads,
                              int32_t head_dim, int32_t dtype, void* store, void* stream) {
  skv_status st;
  if ((st = check_ptr(k_text)) != SKV_OK) return st;
  if ((st = check_ptr(v_text)) != SKV_OK) return st;
  if ((st = check_store(store)) != SKV_OK) return st;
  TextLayout L;
  if ((st = text_layout(n_text, heads, head_dim, dtype, &L)) != SKV_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  char* vdst = (char*)store + L.vt_off;
  if (dtype != SKV_BF16) {
    if (gate([&] { return hipMemcpyAsync(store, k_text, (size_t)L.k_bytes, hipMemcpyDeviceToDevice, s); }) !=
        hipSuccess)
      return SKV_ERR_HIP;
    return gate([&] { return hipMemcpyAsync(vdst, v_text, (size_t)L.k_bytes, hipMemcpyDeviceToDevice, s); }) ==
                   hipSuccess
               ? SKV_OK
               : SKV_ERR_HIP;
  }
  // one launch: keys -> head-major rows [h][key][d], values -> V^T tiles; keys past n_text zero
  // up to the padded length
  skv::WriteArgs wa{};
  wa.k_src = k_text;
  wa.k_dst = store;
  wa.k_hs = L.pad * head_dim;
  wa.v_src = v_text;
  wa.tok_stride = (int64_t)heads * head_dim;
  wa.head_stride = head_dim;
  wa.vt_dst = vdst;
  wa.vt_hs = (int64_t)head_dim * L.pad;
  wa.vt_bs = (int64_t)skv::kVtKeys * head_dim;
  wa.vt_ds = skv::kVtKeys;
  wa.nruns = 0;
  wa.F = n_text;
  wa.H = heads;
  wa.D = head_dim;
  wa.n_tok = n_text;
  wa.row_pad = (int32_t)L.pad;
  return gate([&] { return skv::launch_write_kv(wa, 2, s); }) == hipSuccess ? SKV_OK : SKV_ERR_HIP;
}

skv_status cross_attention_cached(const void* q, int32_t n_q, const void* store, int32_t n_text, int32_t heads,
                                  int32_t head_dim, int32_t dtype, void* out, void* stream) {
  skv_status st;
  if ((st = check_ptr(q)) != SKV_OK) return st;
  if ((st = check_ptr(out)) != SKV_OK) return st;
  if ((st = check_store(store)) != SKV_OK) return st;
  TextLayout L;
  if ((st = text_layout(n_text, heads, head_dim, dtype, &L)) != SKV_OK) return st;
  if (n_q < 1 || (int64_t)n_q * heads > (int64_t)INT32_MAX / 2) return SKV_ERR_SHAPE;
  if (dtype == SKV_BF16 && ((int64_t)n_q + 64) * heads * head_dim * 2 > INT32_MAX) return SKV_ERR_SHAPE;
  const char* vsrc = (const char*)store + L.vt_off;
  const hipStream_t s = (hipStream_t)stream;
  skv::AttnBatch ab{};
  ab.nb = 1;
  skv::AttnArgs& a = ab.b[0];
  a.q = q;
  a.out = out;
  a.alt_seg = 1 << 20;
  a.Lq = n_q;
  a.H = heads;
  a.sl2 = softmax_scale_log2(head_dim);
  a.nseg = 1;
  for (int i = 1; i < 4; ++i) a.seg[i] = skv::KvSeg{nullptr, nullptr, 0, 0, 0, 0, 0, 0, 0, 0};
  if (dtype == SKV_BF16) {
    // K head-major rows of L.pad keys per head; V^T tiles of L.pad keys per head
    a.seg[0] = skv::KvSeg{store, vsrc, L.pad * head_dim, (int64_t)head_dim, (int64_t)head_dim * L.pad, 1,
                          skv::kVtKeys, n_text, 1, 0};
    return gate([&] { return skv::launch_attention_bf16_vt(ab, head_dim, s); }) == hipSuccess ? SKV_OK : SKV_ERR_HIP;
  }
  a.seg[0] = skv::KvSeg{store, vsrc, (int64_t)head_dim, (int64_t)heads * head_dim, (int64_t)head_dim,
                        (int64_t)heads * head_dim, 1, n_text, 0};
  return gate([&] { return skv::launch_attention_f32(a, head_dim, s); }) == hipSuccess ? SKV_OK : SKV_ERR_HIP;
}

// Many-chunk attention: checks shared by the size query and the call.
static skv_status block_causal_geometry(const skv_config* cfg, int32_t n_frames, int32_t q_frame0,
                                        skv::Geometry* g, int64_t* row_pad) {
  skv_status st = skv::make_geometry(cfg, g);
  if (st != SKV_OK) return st;
  if (g->dtype != SKV_BF16) return SKV_ERR_CONFIG;
  if (n_frames < 1) return SKV_ERR_SHAPE;
  // q_frame0 < 0: size query only (no query frames to check)
  if (q_frame0 >= 0 && (q_frame0 >= n_frames || (n_frames - q_frame0) % g->c)) return SKV_ERR_SHAPE;
  const int64_t keys = (int64_t)n_frames * g->F;
  *row_pad = (keys + 63) / 64 * 64;
  // 32-bit offsets inside one head's key rows (token-major) and V^T rows
  if ((keys + 64) * g->H * g->D * g->elt > INT32_MAX || (int64_t)g->D * *row_pad * g->elt > INT32_MAX ||
      keys > INT32_MAX / 2)
    return SKV_ERR_SHAPE;
  return SKV_OK;
}

skv_status block_causal_workspace_bytes(const skv_config* cfg, int32_t n_frames, size_t* bytes) {
  if (!bytes) return SKV_ERR_NULL;
  skv::Geometry g;
  int64_t row_pad = 0;
  const skv_status st = block_causal_geometry(cfg, n_frames, -1, &g, &row_pad);
  if (st != SKV_OK) return st;
  *bytes = (size_t)g.H * g.D * row_pad * g.elt;
  return SKV_OK;
}

skv_status block_causal_attention(const skv_config* cfg, const void* q, const void* k, const void* v,
                                  int32_t n_frames, int32_t q_frame0, void* workspace, void* out, void* stream) {
  skv_status st;
  for (const void* p : {q, k, v, (const void*)workspace, (const void*)out})
    if ((st = check_ptr(p)) != SKV_OK) return st;
  skv::Geometry g;
  int64_t row_pad = 0;
  if (q_frame0 < 0) return SKV_ERR_SHAPE;
  if ((st = block_causal_geometry(cfg, n_frames, q_frame0, &g, &row_pad)) != SKV_OK) return st;
  // values -> V^T rows of the whole sequence in the workspace
  skv::WriteArgs wa{};
  wa.k_src = nullptr;
  wa.v_src = v;
  wa.tok_stride = (int64_t)g.H * g.D;
  wa.head_stride = g.D;
  wa.vt_dst = workspace;
  set_vt(wa, g, row_pad);
  wa.nruns = 0;
  wa.F = g.F;
  wa.H = g.H;
  wa.D = g.D;
  wa.n_tok = n_frames * g.F;
  wa.row_pad = (int32_t)row_pad;
  if (gate([&] { return skv::launch_write_kv(wa, g.elt, (hipStream_t)stream); }) != hipSuccess) return SKV_ERR_HIP;
  skv::AttnBatch ab{};
  ab.nb = 1;
  skv::AttnArgs& a = ab.b[0];
  a.q = q;
  a.out = out;
  a.alt_seg = 1 << 20;
  a.Lq = (n_frames - q_frame0) * g.F;
  a.H = g.H;
  a.sl2 = softmax_scale_log2(g.D);
  a.nseg = 1;
  a.seg[0] = skv::KvSeg{k, workspace, (int64_t)g.D, (int64_t)g.H * g.D, (int64_t)g.D * row_pad, 1, skv::kVtKeys,
                        n_frames * g.F, 1, 0};
  for (int i = 1; i < 4; ++i) a.seg[i] = skv::KvSeg{nullptr, nullptr, 0, 0, 0, 0, 0, 0, 0, 0};
  a.mF = g.F;
  a.mq0 = q_frame0;
  a.mc = g.c;
  a.mS = g.S;
  a.mW = g.W;
  return gate([&] { return skv::launch_attention_bf16_masked(ab, g.D, (hipStream_t)stream); }) == hipSuccess
             ? SKV_OK
             : SKV_ERR_HIP;
}

skv_status sampler_step(const void* x_t, const void* v_cond, const void* v_uncond, double cfg_scale,
                        const void* noise, int64_t n, double sigma, double sigma_next, int32_t dtype, void* x0_out,
                        void* x_next_out, void* stream) {
  skv_status st;
  if ((st = check_ptr(x_t)) != SKV_OK) return st;
  if ((st = check_ptr(v_cond)) != SKV_OK) return st;
  if (!x0_out && !x_next_out) return SKV_ERR_NULL;
  if (x_next_out && !noise) return SKV_ERR_NULL;
  const void* opt[4] = {v_uncond, noise, x0_out, x_next_out};
  for (const void* q : opt)
    if (q && ((uintptr_t)q & 15)) return SKV_ERR_ALIGN;
  if (dtype != SKV_F32 && dtype != SKV_BF16) return SKV_ERR_CONFIG;
  if (!std::isfinite(cfg_scale) || !std::isfinite(sigma) || !std::isfinite(sigma_next)) return SKV_ERR_CONFIG;
  if (n < 0) return SKV_ERR_SHAPE;
  if (n == 0) return SKV_OK;
  skv::SamplerArgs a{x_t, v_cond, v_uncond, x_next_out ? noise : nullptr, x0_out, x_next_out, n,
                     cfg_scale, sigma, sigma_next};
  return gate([&] { return skv::launch_sampler(a, dtype == SKV_BF16 ? 2 : 4, (hipStream_t)stream); }) == hipSuccess ? SKV_OK
                                                                                             : SKV_ERR_HIP;
}

skv_status kv_cache_gather(const skv_cache* cc, void* k_out, void* v_out, int64_t* frame_ids_host, void* stream) {
  skv_cache* c = const_cast<skv_cache*>(cc);
  skv_status st = check_handle(c);
  if (st != SKV_OK) return st;
  if ((st = check_ptr(k_out)) != SKV_OK) return st;
  if ((st = check_ptr(v_out)) != SKV_OK) return st;
  const skv::Geometry& g = c->g;
  const int n = c->ring.n_cached(g);
  for (int i = 0; i < n && frame_ids_host; ++i) frame_ids_host[i] = c->ring.cached_frame(g, i);
  if (n == 0) return SKV_OK;
  skv::FrameRun runs[3];
  int nruns = 0;
  for (int i = 0; i < n; ++i) {
    const int slot = c->ring.slot_of(g, c->ring.cached_frame(g, i));
    if (nruns > 0 && runs[nruns - 1].src0 + runs[nruns - 1].count == slot) {
      ++runs[nruns - 1].count;
    } else {
      if (nruns == 3) return SKV_ERR_STATE;  // cannot happen: sinks + at most two ring runs
      runs[nruns++] = skv::FrameRun{i, 1, slot, i};
    }
  }
  const skv::TokView src[2] = {store_view(g, c->k_store), store_view(g, c->k_store)};
  const skv::TokView dst[2] = {token_view(g, k_out), token_view(g, k_out)};
  st = launched(c, gate([&] {
                  return skv::launch_copy_frames(src, dst, 1, runs, nruns, n, g.F, g.H, g.D, g.elt, (hipStream_t)stream);
                }));
  if (st != SKV_OK) return st;
  skv::WriteArgs va{};
  va.k_dst = v_out;
  va.tok_stride = (int64_t)g.H * g.D;
  va.head_stride = g.D;
  va.vt_dst = c->v_store;
  set_vt(va, g, vt_row(g));
  for (int i = 0; i < 3; ++i)
    va.runs[i] = i < nruns ? skv::FrameRun{runs[i].start, runs[i].count, 0, runs[i].src0} : skv::FrameRun{0, 0, 0, 0};
  va.nruns = nruns;
  va.F = g.F;
  va.H = g.H;
  va.D = g.D;
  va.n_tok = n * g.F;
  va.row_pad = 0;
  return launched(c, gate([&] { return skv::launch_vt_to_tok(va, g.elt, (hipStream_t)stream); }));
}

skv_status kv_cache_restore(skv_cache* c, const void* k, const void* v, const int64_t* frame_ids_host,
                            int32_t n_frames, void* stream) {
  skv_status st = check_handle(c);
  if (st != SKV_OK) return st;
  if (n_frames < 0) return SKV_ERR_SHAPE;
  const skv::Geometry& g = c->g;
  skv::RingState r;
  if (n_frames > 0) {
    if ((st = check_ptr(k)) != SKV_OK) return st;
    if ((st = check_ptr(v)) != SKV_OK) return st;
    if (!frame_ids_host) return SKV_ERR_NULL;
    // the ids must be exactly the ones kv_cache_gather reports for T = last id + 1
    if (frame_ids_host[n_frames - 1] < 0) return SKV_ERR_SHAPE;
    r.T = frame_ids_host[n_frames - 1] + 1;
    if (r.n_cached(g) != n_frames) return SKV_ERR_SHAPE;
    for (int i = 0; i < n_frames; ++i)
      if (frame_ids_host[i] != r.cached_frame(g, i)) return SKV_ERR_SHAPE;
    // logical frame i -> its slot, merged into runs of consecutive slots (sinks, ring part a, ring part b)
    skv::FrameRun runs[3];
    int nruns = 0;
    for (int i = 0; i < n_frames; ++i) {
      const int slot = r.slot_of(g, frame_ids_host[i]);
      if (nruns > 0 && runs[nruns - 1].dst0 + runs[nruns - 1].count == slot) {
        ++runs[nruns - 1].count;
      } else {
        if (nruns == 3) return SKV_ERR_STATE;  // cannot happen: sinks + at most two ring runs
        runs[nruns++] = skv::FrameRun{i, 1, i, slot};
      }
    }
    // the bytes go back as they were gathered (keys stay as stored: rotated or raw), K rows + V^T
    skv::WriteArgs wa{};
    wa.k_src = k;
    wa.v_src = v;
    wa.tok_stride = (int64_t)g.H * g.D;
    wa.head_stride = g.D;
    wa.k_dst = c->k_store;
    wa.k_hs = (int64_t)g.W * g.F * g.D;
    wa.vt_dst = c->v_store;
    set_vt(wa, g, vt_row(g));
    for (int i = 0; i < 3; ++i) wa.runs[i] = i < nruns ? runs[i] : skv::FrameRun{0, 0, 0, 0};
    wa.nruns = nruns;
    wa.F = g.F;
    wa.H = g.H;
    wa.D = g.D;
    wa.n_tok = n_frames * g.F;
    wa.row_pad = 0;
    st = launched(c, gate([&] { return skv::launch_write_kv(wa, g.elt, (hipStream_t)stream); }));
    if (st != SKV_OK) return st;
  }
  c->ring.T = r.T;
  c->window_ready = false;
  c->v_staged = false;
  return SKV_OK;
}

void skv_debug_fail_launches(int32_t n) { g_fail_launches.store(n > 0 ? n : 0); }

}  // extern "C"
