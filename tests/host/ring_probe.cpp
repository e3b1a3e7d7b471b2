// Host-only driver of the ring bookkeeping (skv_core.cpp) for CPU tests.
// stdin:  "cfg S W c" once, then "append n" lines.
// stdout: one JSON object per append: slots written, cached frames with their
//         slots, and the visible-set plan a chunk of c frames would use.
#include <cstdio>
#include <cstring>
#include <string>

#include "../../streaming_kv_cache_amd/csrc/skv_core.hpp"

int main() {
  char cmd[32];
  int S = 0, W = 0, c = 0;
  if (scanf("%31s %d %d %d", cmd, &S, &W, &c) != 4 || strcmp(cmd, "cfg") != 0) return 2;
  skv_config cfg{};
  cfg.heads = 1;
  cfg.head_dim = 64;
  cfg.grid_h = 1;
  cfg.grid_w = 1;
  cfg.chunk_frames = c;
  cfg.sink_frames = S;
  cfg.window_frames = W;
  cfg.dtype = SKV_BF16;
  cfg.rope_mode = SKV_ROPE_ABS;
  skv::Geometry g;
  skv_status st = skv::make_geometry(&cfg, &g);
  if (st != SKV_OK) {
    printf("{\"error\": %d}\n", (int)st);
    return 0;
  }
  skv::RingState ring;
  int n = 0;
  while (scanf("%31s %d", cmd, &n) == 2) {
    std::string out = "{\"slots\": [";
    for (int i = 0; i < n; ++i) out += (i ? ", " : "") + std::to_string(ring.slot_of(g, ring.T + i));
    ring.T += n;
    out += "], \"T\": " + std::to_string(ring.T) + ", \"cached\": [";
    const int nc = ring.n_cached(g);
    for (int i = 0; i < nc; ++i) {
      const long long f = ring.cached_frame(g, i);
      out += (i ? ", [" : "[") + std::to_string(f) + ", " + std::to_string(ring.slot_of(g, f)) + "]";
    }
    const skv::VisiblePlan p = ring.plan(g, g.c);
    out += "], \"n_vis\": " + std::to_string(p.n_vis) + ", \"n_hist\": " + std::to_string(p.n_hist) + ", \"runs\": [";
    for (int i = 0; i < p.n_runs; ++i)
      out += (i ? ", [" : "[") + std::to_string(p.runs[i].slot0) + ", " + std::to_string(p.runs[i].frames) +
             ", " + std::to_string(p.runs[i].logical0) + "]";
    out += "]}";
    puts(out.c_str());
  }
  return 0;
}
