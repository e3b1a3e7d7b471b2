// Many-chunk block-causal attention with its workspace in library-owned static device memory,
// for callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The workspace (the values of the sequence transposed to V^T rows) lives
// in a file-scope __device__ array; each device that runs this holds its own copy, whose address is
// looked up once per device with that device current and kept.  Calls that overlap on one device
// share that array and race; every byte a call reads from it is written by the same call first
// (the V^T rows, their zero padding included), so nothing has to start at zero.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/skv.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch` (looked up on the first call per device).
skv_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SKV_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SKV_OK;
}

}  // namespace

extern "C" skv_status block_causal_attention_noalloc(const skv_config* cfg, const void* q, const void* k,
                                                     const void* v, int32_t n_frames, int32_t q_frame0, void* out,
                                                     void* stream) {
  size_t need = 0;
  skv_status st = block_causal_workspace_bytes(cfg, n_frames, &need);
  if (st != SKV_OK) return st;
  if (need > (size_t)SKV_NOALLOC_SCRATCH_BYTES) return SKV_ERR_SHAPE;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != SKV_OK) return st;
  return block_causal_attention(cfg, q, k, v, n_frames, q_frame0, ws, out, stream);
}
