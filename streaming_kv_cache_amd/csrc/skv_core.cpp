// Configuration checks and the visible-set plan (see skv_core.hpp).
#include "skv_core.hpp"

#include <cmath>
#include <climits>

namespace skv {

bool attention_head_dim_supported(int32_t dtype, int32_t D) {
  if (dtype == SKV_BF16) return D == 64 || D == 128;
  if (dtype == SKV_F32) return D == 32 || D == 64 || D == 128;
  return false;
}

skv_status make_geometry(const skv_config* cfg, Geometry* g) {
  if (!cfg || !g) return SKV_ERR_NULL;
  Geometry r;
  r.H = cfg->heads;
  r.D = cfg->head_dim;
  r.gh = cfg->grid_h;
  r.gw = cfg->grid_w;
  r.c = cfg->chunk_frames;
  r.S = cfg->sink_frames;
  r.W = cfg->window_frames;
  if (r.H <= 0 || r.D <= 0 || r.gh <= 0 || r.gw <= 0 || r.c <= 0 || r.S < 0) return SKV_ERR_CONFIG;
  if ((int64_t)r.gh * r.gw > (1 << 24)) return SKV_ERR_CONFIG;
  r.F = r.gh * r.gw;
  if ((int64_t)r.W < (int64_t)r.S + r.c) return SKV_ERR_CONFIG;
  if ((int64_t)r.W * r.F > INT32_MAX / 2) return SKV_ERR_CONFIG;
  if ((int64_t)r.H * r.D > 65536) return SKV_ERR_CONFIG;
  r.R = r.W - r.S;
  if (cfg->dtype != SKV_F32 && cfg->dtype != SKV_BF16) return SKV_ERR_CONFIG;
  r.dtype = cfg->dtype;
  r.elt = r.dtype == SKV_BF16 ? 2 : 4;
  if (!attention_head_dim_supported(r.dtype, r.D)) return SKV_ERR_CONFIG;
  if (r.dtype == SKV_BF16) {
    // the bf16 attention kernel addresses each head's key range with 32-bit byte offsets:
    // the current chunk (token-major rows of H*D), the stores' rows, and V^T rows of W*F keys
    const int64_t lim = INT32_MAX;
    const int64_t cur = ((int64_t)r.c * r.F + 64) * r.H * r.D * r.elt;
    const int64_t kst = ((int64_t)r.W * r.F + 64) * r.D * r.elt;
    const int64_t vst = (int64_t)r.D * ((int64_t)r.W * r.F + 64) * r.elt;
    if (cur > lim || kst > lim || vst > lim) return SKV_ERR_CONFIG;
  }
  if (cfg->rope_mode != SKV_ROPE_ABS && cfg->rope_mode != SKV_ROPE_REL) return SKV_ERR_CONFIG;
  if (cfg->fused_rope != 0 && cfg->fused_rope != 1) return SKV_ERR_CONFIG;
  r.fused = cfg->fused_rope;
  r.mode = cfg->rope_mode;
  if (cfg->rope_t == 0 && cfg->rope_h == 0 && cfg->rope_w == 0) {
    int32_t hw = 2 * (r.D / 6);
    r.rope_t = r.D - 2 * hw;
    r.rope_h = hw;
    r.rope_w = hw;
  } else {
    r.rope_t = cfg->rope_t;
    r.rope_h = cfg->rope_h;
    r.rope_w = cfg->rope_w;
  }
  if (r.rope_t < 0 || r.rope_h < 0 || r.rope_w < 0) return SKV_ERR_CONFIG;
  if ((r.rope_t | r.rope_h | r.rope_w) & 1) return SKV_ERR_CONFIG;
  if (r.rope_t + r.rope_h + r.rope_w != r.D) return SKV_ERR_CONFIG;
  double th = cfg->rope_theta == 0.0 ? 10000.0 : cfg->rope_theta;
  if (!(th > 0.0) || !std::isfinite(th)) return SKV_ERR_CONFIG;
  r.theta = th;
  *g = r;
  return SKV_OK;
}

VisiblePlan RingState::plan(const Geometry& g, int32_t chunk) const {
  VisiblePlan p;
  p.n_sink_vis = (int32_t)(T < g.S ? T : g.S);
  int64_t ring_avail = T > g.S ? T - g.S : 0;
  if (ring_avail > g.R) ring_avail = g.R;
  int64_t room = (int64_t)g.W - g.S - chunk;  // history frames after the sinks that still fit
  if (room < 0) room = 0;
  p.n_ring_vis = (int32_t)(ring_avail < room ? ring_avail : room);
  p.n_hist = p.n_sink_vis + p.n_ring_vis;
  p.n_vis = p.n_hist + chunk;
  p.first_ring_frame = T - p.n_ring_vis;
  if (p.n_sink_vis > 0) {
    p.runs[p.n_runs++] = SlotRun{0, p.n_sink_vis, 0};
  }
  if (p.n_ring_vis > 0) {
    int32_t start = slot_of(g, p.first_ring_frame);
    p.ring_start = start;
    int32_t a = g.W - start;
    if (a > p.n_ring_vis) a = p.n_ring_vis;
    p.runs[p.n_runs++] = SlotRun{start, a, p.n_sink_vis};
    if (a < p.n_ring_vis) p.runs[p.n_runs++] = SlotRun{g.S, p.n_ring_vis - a, p.n_sink_vis + a};
  }
  return p;
}

}  // namespace skv
