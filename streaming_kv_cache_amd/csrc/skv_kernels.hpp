// Internal launch interface between the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "skv_device.hpp"

namespace skv {

// Copy n_frames whole frames of n_tensors (1 or 2) token views from src to dst.
hipError_t launch_copy_frames(const TokView src[2], const TokView dst[2], int n_tensors, const FrameRun* runs,
                              int nruns, int n_frames, int F, int H, int D, int elt, hipStream_t stream);

// Write-back of whole frames (K rows + transposed V) and current-chunk staging.
// Sources are token-major [tokens, H, D] (token t, head h at t*tok_stride + h*head_stride).
// K store: head h, key j at k_dst + h*k_hs + j*D.  V^T: (h, d, key j) at vt_dst + h*vt_hs +
// (j / 64)*vt_bs + d*vt_ds + j % 64 (bf16 tiles: vt_bs = 64*D, vt_ds = 64; fp32 rows:
// vt_bs = 64, vt_ds = row length).  runs map launch frames to their key-space frame (slot) in
// dst0, and the launch's workgroups cover the 64-key tiles of those key ranges (whole tiles
// are written as contiguous blocks); nruns == 0 means key = token, and V^T is written
// (zero-filled) up to row_pad keys.  k_src == nullptr writes V only.  vt_to_tok reads vt_dst
// and writes token-major rows to k_dst.
struct WriteArgs {
  const void* k_src;
  const void* v_src;
  int64_t tok_stride, head_stride;
  void* k_dst;
  int64_t k_hs;
  void* vt_dst;
  int64_t vt_hs, vt_ds, vt_bs;
  FrameRun runs[3];
  int32_t nruns;
  int32_t F, H, D;
  int32_t n_tok;
  int32_t row_pad;
  // filled by launch_write_kv for nruns > 0: run r covers 64-key tiles tile0[r] ... and the
  // launch's workgroups [tile_pre[r], tile_pre[r + 1])
  int32_t tile0[3], tile_pre[4];
};
hipError_t launch_write_kv(const WriteArgs& a, int elt, hipStream_t stream);

struct SamplerArgs {
  const void* x_t;
  const void* v_cond;
  const void* v_uncond;  // NULL: no guidance
  const void* noise;     // read only when x_next_out is set
  void* x0_out;          // NULL: not written
  void* x_next_out;      // NULL: not written (last step)
  int64_t n;
  double cfg_scale, sigma, sigma_next;
};
hipError_t launch_sampler(const SamplerArgs& a, int elt, hipStream_t stream);
hipError_t launch_vt_to_tok(const WriteArgs& a, int elt, hipStream_t stream);

// One tensor of a rotary launch: src -> dst at time ids t0 + frame (clamped to [0, clamp_max] if >= 0).
struct RopeJob {
  TokView src, dst;
  int64_t t0;
  int32_t clamp_max;
};
// Up to three tensors with the same frames, grid and split share one launch (grid z = job).
struct RopeLaunch {
  RopeJob job[3];
  int njobs;
  FrameRun runs[3];
  int nruns;
  int n_frames, F, gw, H, D;
  int rope_t, rope_h, rope_w;
  double theta;
  bool dtype_bf16;
};
hipError_t launch_rope(const RopeLaunch& L, hipStream_t stream);
// bf16, D in {64, 128}: the rotary launch L and the staging write w (nruns == 0) as one grid.
hipError_t launch_prepare_pass(const RopeLaunch& L, const WriteArgs& w, hipStream_t stream);

// softmax(q K^T * scale) V over the concatenated key ranges of a.seg.
// bf16, V transposed (cache path) / V token-major (cross attention); fp32 takes any V strides.
hipError_t launch_attention_bf16_vt(const AttnBatch& ab, int D, hipStream_t stream);
hipError_t launch_attention_bf16_masked(const AttnBatch& ab, int D, hipStream_t stream);
hipError_t launch_attention_bf16_tokv(const AttnArgs& a, int D, hipStream_t stream);
hipError_t launch_attention_f32(const AttnArgs& a, int D, hipStream_t stream);

}  // namespace skv
