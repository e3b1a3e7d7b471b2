// Internal launch interface between the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "skv_device.hpp"

namespace skv {

// Copy n_frames whole frames of K (index 0) and V (index 1) from src to dst views.
hipError_t launch_copy_frames(const TokView src[2], const TokView dst[2], const FrameRun* runs, int nruns,
                              int n_frames, int F, int H, int D, int elt, hipStream_t stream);

struct RopeLaunch {
  TokView src, dst;
  FrameRun runs[3];
  int nruns;
  int n_frames, F, gw, H, D;
  int rope_t, rope_h, rope_w;
  double theta;
  int64_t t0;
  int clamp_max;
  bool dtype_bf16;
};
hipError_t launch_rope(const RopeLaunch& L, hipStream_t stream);

// softmax(q K^T * scale) V over the concatenated key ranges of a.seg.
hipError_t launch_attention_bf16(const AttnArgs& a, int D, hipStream_t stream);
hipError_t launch_attention_f32(const AttnArgs& a, int D, hipStream_t stream);

}  // namespace skv
